// Shape-keyed dispatch table: measured best (variant, split, M-split) per
// problem shape on MI355X.  Entries live in bsmm_tuned_table.inc, which the
// tuning sweep writes; the key is (op, out dtype, G, M, N, K) and must be
// unique (checked by the CPU tests).
#pragma once

namespace bsmm {

struct TunedEntry {
  int op;               // bsmm_op
  int out_dtype;        // bsmm_dtype
  int G, M, N, K;
  const char* variant;  // main launch
  int split;            // K slices of the main launch
  int m_split;          // rows of the bulk launch (0: no M-split)
  const char* tail_variant;  // "" when m_split == 0
  int tail_split;       // K slices of the tail launch (1: none)
};

const TunedEntry* tuned_table(int* count);

}  // namespace bsmm
