// Decode kernels instantiated for 7 query heads per KV head (one
// translation unit per group size keeps builds parallel).
#include "decode_kernels.h"

template int leank::launch_decode<7, 0>(const leank::DecodeParams&, int64_t, int64_t,
                                             int, hipStream_t);
template int leank::launch_decode<7, 4>(const leank::DecodeParams&, int64_t, int64_t,
                                             int, hipStream_t);
template int leank::launch_decode<7, 8>(const leank::DecodeParams&, int64_t, int64_t,
                                             int, hipStream_t);
