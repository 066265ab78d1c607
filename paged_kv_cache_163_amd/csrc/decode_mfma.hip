// Split-partition paged decode on the gfx950 matrix cores: the kernel and its
// launcher.  The work of a work-group is decode_wg (decode_mfma.h).
#include "decode_mfma.h"

namespace pa {
namespace {

template <int D, int M, int NW, bool WP>
__global__ __launch_bounds__(NW * 64)
#if PA_MFMA_MIN_WAVES_PER_EU > 0
__attribute__((amdgpu_waves_per_eu(PA_MFMA_MIN_WAVES_PER_EU)))
#endif
void decode_mfma_kernel(DecodeParams p) {
  __shared__ DecodeLds<D, NW> lds;
  decode_wg<D, M, NW, WP>(p, blockIdx.x, lds);
}

template <int D, int NW, bool WP>
hipError_t launch_nw(const DecodeParams& p, int mode, dim3 grid, hipStream_t stream) {
  const dim3 block(NW * 64);
  if (mode == kModeLayered)
    decode_mfma_kernel<D, kModeLayered, NW, WP><<<grid, block, 0, stream>>>(p);
  else if (mode == kModeOrdered)
    decode_mfma_kernel<D, kModeOrdered, NW, WP><<<grid, block, 0, stream>>>(p);
  else
    decode_mfma_kernel<D, kModePlain, NW, WP><<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, int mode, dim3 grid, hipStream_t stream) {
  if (mode == kModeFused || mode == kModeFusedOrdered) {
    // the fused append keeps one partition per work-group
    const dim3 block(p.waves * 64);
    if (p.wave_parts || (p.waves != 4 && p.waves != 2)) return hipErrorInvalidValue;
    if (mode == kModeFused) {
      if (p.waves == 4)
        decode_mfma_kernel<D, kModeFused, 4, false><<<grid, block, 0, stream>>>(p);
      else
        decode_mfma_kernel<D, kModeFused, 2, false><<<grid, block, 0, stream>>>(p);
    } else {
      if (p.waves == 4)
        decode_mfma_kernel<D, kModeFusedOrdered, 4, false><<<grid, block, 0, stream>>>(p);
      else
        decode_mfma_kernel<D, kModeFusedOrdered, 2, false><<<grid, block, 0, stream>>>(p);
    }
    return hipGetLastError();
  }
  if (p.wave_parts) {
    if (p.waves != 4) return hipErrorInvalidValue;
    return launch_nw<D, 4, true>(p, mode, grid, stream);
  }
  switch (p.waves) {
    case 2: return launch_nw<D, 2, false>(p, mode, grid, stream);
    case 4: return launch_nw<D, 4, false>(p, mode, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  // with wave-per-partition work-groups, one work-group covers `waves` partitions
  const int64_t groups = p.wave_parts ? (p.num_partitions + p.waves - 1) / p.waves
                                      : p.num_partitions;
  const dim3 grid((unsigned)(groups * p.num_seqs * p.kv_heads),
                  (unsigned)(p.num_layers > 1 ? p.num_layers : 1));
  const int mode = p.block_stride != 0     ? kModeLayered
                   : p.new_slots != nullptr ? (p.order != nullptr ? kModeFusedOrdered : kModeFused)
                   : p.order != nullptr     ? kModeOrdered
                                            : kModePlain;
  if (head_dim == 128) return launch_d<128>(p, mode, grid, stream);
  if (head_dim == 64) return launch_d<64>(p, mode, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
