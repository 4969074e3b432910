// Small kernels outside the head's hot path: the sampler's random numbers as the kernels
// draw them (for checking the generator), and the reset of the batched selection's
// per-cluster state before a selection that no stage-1 launch has prepared.
#include "fh_device.h"
#include "fh_internal.h"

namespace fh {

// words[i] = Philox word of element n0 + i of (row, stream) under g; gumbel[i] = G(u) in fp32,
// through the same device functions the forward's keys use.
__global__ __launch_bounds__(256) void k_philox_words(Rng g, uint32_t row, uint32_t stream, uint32_t n0,
                                                      int64_t count, uint32_t* words, float* gum) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    const uint32_t w = rng_word(g, row, stream, n0 + (uint32_t)i);
    if (words) words[i] = w;
    if (gum) gum[i] = gumbel(word_to_uniform(w));
  }
}

hipError_t launch_philox_words(uint64_t seed, uint32_t row, uint64_t step, uint32_t stream, uint32_t n0,
                               int64_t count, uint32_t* words, float* gum, hipStream_t st) {
  int64_t wgs = (count + 255) / 256;
  if (wgs > 65536) wgs = 65536;
  hipLaunchKernelGGL(k_philox_words, dim3((unsigned)wgs), dim3(256), 0, st, make_rng(seed, step), row, stream, n0,
                     count, words, gum);
  return hipGetLastError();
}

// Clears the row masks [c][W], the kept flags [c] and the kept-cluster count of a B > 1
// workspace (what the stage-1 kernels clear on the way).
__global__ __launch_bounds__(256) void k_clear_select(uint64_t* mask, int nmask, uint32_t* kflag, int c,
                                                      int32_t* nkept) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nmask) mask[i] = 0ull;
  if (i < c) kflag[i] = 0u;
  if (i == 0) *nkept = 0;
}

hipError_t launch_clear_select(const Workspace& ws, int c, hipStream_t st) {
  if (!ws.mask) return hipSuccess;
  const int n = c * ws.W > c ? c * ws.W : c;
  hipLaunchKernelGGL(k_clear_select, dim3((n + 255) / 256), dim3(256), 0, st, ws.mask, c * ws.W, ws.kflag, c,
                     ws.nkept);
  return hipGetLastError();
}

}  // namespace fh
