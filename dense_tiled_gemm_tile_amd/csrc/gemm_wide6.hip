// Wide streaming GEMM instances for 6-bit operands (e2m3, e3m2) on the
// 32x32x64 scaled MFMA, on the 8-bit schedule (a stage is 128 k, 96 bytes of
// each row): 57/58 without block scales, 59/60 applying them.
#include "gemm_wide.h"

#define TG_WIDE6_LIST(X)                           \
    X(57, TG_E2M3, 4, 5, 16, 1, 1, 17, 16, 100)        \
    X(58, TG_E3M2, 4, 5, 16, 1, 1, 17, 16, 100)        \
    X(59, TG_E2M3, 4, 5, 16, 1, 1, 81, 16, 90)         \
    X(60, TG_E3M2, 4, 5, 16, 1, 1, 81, 16, 90)

TG_WIDE6_LIST(TG_INSTANTIATE_WIDE)

#ifndef __HIP_DEVICE_COMPILE__
extern const TgKernelDesc tg_entries_wide6[] = {TG_WIDE6_LIST(TG_ENTRY_WIDE)};
extern const int tg_entries_wide6_count = sizeof(tg_entries_wide6) / sizeof(tg_entries_wide6[0]);
#endif  // __HIP_DEVICE_COMPILE__
