// ffd_kernels_stream.hip -- the streaming-policy decode kernels (decode_kernel<..., STREAM = true>)
// and their launchers: the second half of ffd_kernels.hip, compiled as a translation unit of its
// own so that the two halves build in parallel.
#define FFD_PART 1
#include "ffd_kernels.hip"
