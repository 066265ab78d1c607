// Split-partition paged decode on the gfx950 matrix cores: the kernel and its
// launcher.  The work of a work-group is decode_wg (decode_mfma.h).
#include "decode_mfma.h"

namespace pa {
namespace {

template <int D, int M>
__global__ __launch_bounds__(kWaves * 64)
#if PA_MFMA_MIN_WAVES_PER_EU > 0
__attribute__((amdgpu_waves_per_eu(PA_MFMA_MIN_WAVES_PER_EU)))
#endif
void decode_mfma_kernel(DecodeParams p) {
  __shared__ DecodeLds<D> lds;
  decode_wg<D, M>(p, blockIdx.x, lds);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_partitions * p.num_seqs * p.kv_heads),
                  (unsigned)(p.num_layers > 1 ? p.num_layers : 1));
  const dim3 block(kWaves * 64);
  const int mode = p.block_stride != 0     ? kModeLayered
                   : p.new_slots != nullptr ? kModeFused
                   : p.order != nullptr     ? kModeOrdered
                                            : kModePlain;
#define PA_LAUNCH(DIM, MODE) decode_mfma_kernel<DIM, MODE><<<grid, block, 0, stream>>>(p)
  if (head_dim == 128) {
    if (mode == kModeLayered) PA_LAUNCH(128, kModeLayered);
    else if (mode == kModeFused) PA_LAUNCH(128, kModeFused);
    else if (mode == kModeOrdered) PA_LAUNCH(128, kModeOrdered);
    else PA_LAUNCH(128, kModePlain);
  } else if (head_dim == 64) {
    if (mode == kModeLayered) PA_LAUNCH(64, kModeLayered);
    else if (mode == kModeFused) PA_LAUNCH(64, kModeFused);
    else if (mode == kModeOrdered) PA_LAUNCH(64, kModeOrdered);
    else PA_LAUNCH(64, kModePlain);
  } else {
    return hipErrorInvalidValue;
  }
#undef PA_LAUNCH
  return hipGetLastError();
}

}  // namespace pa
