// Wide streaming GEMM instances for 8-bit operands (e4m3, e5m2) on the
// 32x32x64 scaled MFMA; 12/13 apply block scales, 10/11 carry no scale code.
#include "gemm_wide.h"

#define TG_WIDE8_LIST(X)                           \
    X(10, TG_E4M3, 4, 5, 16, 1, 1, 17, 16, 107)        \
    X(11, TG_E5M2, 4, 5, 16, 1, 1, 17, 16, 107)        \
    X(12, TG_E4M3, 4, 5, 16, 1, 1, 81, 16, 90)         \
    X(13, TG_E5M2, 4, 5, 16, 1, 1, 81, 16, 90)

TG_WIDE8_LIST(TG_INSTANTIATE_WIDE)

#ifndef __HIP_DEVICE_COMPILE__
extern const TgKernelDesc tg_entries_wide8[] = {TG_WIDE8_LIST(TG_ENTRY_WIDE)};
extern const int tg_entries_wide8_count = sizeof(tg_entries_wide8) / sizeof(tg_entries_wide8[0]);
#endif  // __HIP_DEVICE_COMPILE__
