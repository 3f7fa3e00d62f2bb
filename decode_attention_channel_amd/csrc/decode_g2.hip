// Decode kernels instantiated for 2 query heads per KV head (one
// translation unit per group size keeps builds parallel).
#include "decode_kernels.h"

template int leank::launch_decode<2, 0>(const leank::DecodeParams&, int64_t, int64_t,
                                             int, hipStream_t);
template int leank::launch_decode<2, 4>(const leank::DecodeParams&, int64_t, int64_t,
                                             int, hipStream_t);
template int leank::launch_decode<2, 8>(const leank::DecodeParams&, int64_t, int64_t,
                                             int, hipStream_t);
