#include "bsmm_tuned.h"

namespace bsmm {

static const TunedEntry kTable[] = {
#include "bsmm_tuned_table.inc"
    {-1, -1, 0, 0, 0, 0, "", 0, 0, "", 1},   // sentinel (never matches)
};

const TunedEntry* tuned_table(int* count) {
  *count = (int)(sizeof(kTable) / sizeof(kTable[0])) - 1;
  return kTable;
}

}  // namespace bsmm
