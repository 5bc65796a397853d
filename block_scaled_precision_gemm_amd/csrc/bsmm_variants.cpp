// The table of kernel configurations compiled into the library, and the
// per-configuration dispatch on (operation, output type).  Host code; the
// kernels themselves are instantiated in the HIP translation units.
#include "bsmm_internal.h"

namespace bsmm {
namespace {

template <int WM, int WN, int RING, bool SK, bool PK, int KIND>
int launch_variant(const Problem& p, const Launch& l) {
  switch (p.op) {
    case BSMM_OP_INT8_ROWWISE:
      if (p.out_dtype == BSMM_I32)
        return launch_kernel<BSMM_OP_INT8_ROWWISE, BSMM_I32, WM, WN, RING, SK, PK, KIND>(p, l);
      if (p.out_dtype == BSMM_F32)
        return launch_kernel<BSMM_OP_INT8_ROWWISE, BSMM_F32, WM, WN, RING, SK, PK, KIND>(p, l);
      return launch_kernel<BSMM_OP_INT8_ROWWISE, BSMM_BF16, WM, WN, RING, SK, PK, KIND>(p, l);
    case BSMM_OP_FP8_BLOCKWISE:
      if (p.out_dtype == BSMM_F32)
        return launch_kernel<BSMM_OP_FP8_BLOCKWISE, BSMM_F32, WM, WN, RING, SK, PK, KIND>(p, l);
      return launch_kernel<BSMM_OP_FP8_BLOCKWISE, BSMM_BF16, WM, WN, RING, SK, PK, KIND>(p, l);
    case BSMM_OP_FP8_MX_BMM:
      if (p.out_dtype == BSMM_F32)
        return launch_kernel<BSMM_OP_FP8_MX_BMM, BSMM_F32, WM, WN, RING, SK, PK, KIND>(p, l);
      return launch_kernel<BSMM_OP_FP8_MX_BMM, BSMM_BF16, WM, WN, RING, SK, PK, KIND>(p, l);
    case BSMM_OP_FP8_MX32_MM:
      if (p.out_dtype == BSMM_F32)
        return launch_kernel<BSMM_OP_FP8_MX32_MM, BSMM_F32, WM, WN, RING, SK, PK, KIND>(p, l);
      return launch_kernel<BSMM_OP_FP8_MX32_MM, BSMM_BF16, WM, WN, RING, SK, PK, KIND>(p, l);
    case BSMM_OP_FP8_GROUPWISE:
      if (p.out_dtype == BSMM_F32)
        return launch_kernel<BSMM_OP_FP8_GROUPWISE, BSMM_F32, WM, WN, RING, SK, PK, KIND>(p, l);
      return launch_kernel<BSMM_OP_FP8_GROUPWISE, BSMM_BF16, WM, WN, RING, SK, PK, KIND>(p, l);
    default:
      if (p.out_dtype == BSMM_F32)
        return launch_kernel<BSMM_OP_FP8_SCALED_MM, BSMM_F32, WM, WN, RING, SK, PK, KIND>(p, l);
      if (p.out_dtype == BSMM_E4M3)
        return launch_kernel<BSMM_OP_FP8_SCALED_MM, BSMM_E4M3, WM, WN, RING, SK, PK, KIND>(p, l);
      return launch_kernel<BSMM_OP_FP8_SCALED_MM, BSMM_BF16, WM, WN, RING, SK, PK, KIND>(p, l);
  }
}

constexpr unsigned kAllOps = 63u;

// name, tile_m, tile_n, ops, masked tail, persistent, packed scales,
// workgroups per CU, unpacked sibling, largest M (the skinny kernel: 16,
// the narrow kernels: 128), kind, launch
const Variant kVariants[] = {
#define BSMM_VARIANT(NAME, TM, TN, WM, WN, RING, SK, PK, WPC, UNPACKED, KIND) \
  {NAME, TM, TN, kAllOps, true, SK, PK, WPC, UNPACKED,                                      \
   KIND == 2 ? 16 : (KIND == 3 || KIND == 4) ? 128 : 0, KIND,                                \
   launch_variant<WM, WN, RING, SK, PK, KIND>},
#include "bsmm_variants.inc"
#undef BSMM_VARIANT
};

}  // namespace

const Variant* variants(int* count) {
  *count = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
  return kVariants;
}

}  // namespace bsmm
