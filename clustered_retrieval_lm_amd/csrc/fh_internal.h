// Internal interface between the C-ABI layer (fh_api.hip) and the kernel launchers
// (fh_kernels.hip).  Launchers enqueue work on a stream and return the launch status;
// every shape and pointer has been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fh {

struct HeadShape {
  int B, d, c, b;     // rows of h, hidden size, clusters, tokens per cluster
  int h_bf16;         // h storage: 1 = bf16, 0 = f32
  int c_fmt;          // RowFmt of the centroids
  int e_fmt;          // RowFmt of the tiles / dense E
};

struct Sampling {
  int sample;         // 0 greedy, 1 sampling
  float tau;
  uint64_t seed, step;
};

// Per-row packed maxima are kBestStride uint64 apart (one 128-byte line per row), so the
// atomic maxima of different rows never contend for a cache line.
constexpr int kBestStride = 16;

// B = 1: the fused selection + stage 2 runs kB1Threads threads per workgroup; the workspace
// keys are padded to b1_key_slots(c) (a multiple of kB1Threads, at least 2 of them).
constexpr int kB1Threads = 1024;
constexpr int kB1Workgroups = 256;
__host__ __device__ inline int b1_key_slots(int c) {
  int s = 2;
  while (s * kB1Threads < c) s *= 2;
  return s * kB1Threads;
}

// B = 1 candidate lists, written by stage 1 and read by the fused selection.  Stage 1 runs one
// workgroup of g / 4 waves per group of g consecutive clusters and lists the m = min(g, 16)
// largest keys of its group in descending order (key desc, id asc) as packed entries
// (ord key << 32 | ~id): group w's entries are lst[w m .. w m + m).  Slots past c in the last
// group hold entries whose high word is 0 (they decode to NaN and rank below every key).  The
// top p of the c keys equals the top p of the L = ngroups m entries unless some group with
// m < g has its m-th entry among those p (then it may hold more); R entries are real keys.
// g = 64 needs 1024-thread workgroups, whose rows fit in registers up to 3 chunk slots; groups
// are chosen large enough to cut the entries, small enough to keep >= 240 workgroups busy.
struct B1Lists {
  int g, m, ngroups, L, R;
};
inline B1Lists b1_lists(int c, int chunk_slots_c) {
  B1Lists l;
  l.g = (chunk_slots_c <= 3 && (c + 63) / 64 >= 240) ? 64 : (c + 31) / 32 >= 240 ? 32 : 16;
  l.m = l.g < 16 ? l.g : 16;
  l.ngroups = (c + l.g - 1) / l.g;
  l.L = l.ngroups * l.m;
  const int last = c - (l.ngroups - 1) * l.g;
  l.R = (l.ngroups - 1) * l.m + (last < l.m ? last : l.m);
  return l;
}

// Workspace carve-up (all offsets 256-byte aligned): keys, masks, best, probes; the
// regions stage 1 writes come first so their offsets do not depend on p.
struct Workspace {
  float* keys;        // [B][c] stage-1 keys
  uint64_t* lst;      // B = 1: the candidate lists (B1Lists), up to c + 64 entries
  int32_t* probes;    // [B][p] kept clusters, ascending
  uint64_t* best;     // [B][kBestStride] packed (key, ~token) maxima (element 0 of each line)
  uint64_t* part;     // [256] per-workgroup maxima of the fused B = 1 stage 2
  uint64_t* mask;     // [c][W] rows that kept cluster k (B > 1 only), W = ceil(B / 64)
  uint32_t* kflag;    // [c] cluster kept by some row (B > 1 only)
  int32_t* klist;     // [c] the clusters kept by any row, in no particular order (B > 1 only)
  int32_t* nkept;     // [1] their count (B > 1 only)
  int W;
  size_t bytes;
};

Workspace carve_workspace(void* base, int B, int c, int p);
size_t dense_workspace_bytes(int B);

// Largest chunk-slot count per lane a row format supports (16-byte chunks, 64 lanes).
int max_chunk_slots(int fmt);
int chunk_slots(int fmt, int d);

hipError_t launch_scores(const HeadShape& s, const void* h, const void* C, const Sampling& smp,
                         const Workspace& ws, float* keys_out, hipStream_t st);
hipError_t launch_select(const HeadShape& s, int p, const Workspace& ws, int32_t* probe_out,
                         hipStream_t st);
hipError_t launch_tiles(const HeadShape& s, int p, const void* h, const int32_t* c2t,
                        const void* tiles, const uint16_t* scales, const Sampling& smp,
                        const Workspace& ws, float* logits_out, int32_t* tokens_out,
                        int32_t* token, hipStream_t st);
// One B = 1 call as the fused kernels (fh_b1.hip) take it.
struct B1Args {
  const void* h;
  const void* C;
  const uint16_t* c_scales;   // int4 centroids: their scales
  int h_bf16, c, d, b, p;
  int sample;
  float tau;
  uint64_t seed, step;
  float* keys;
  float* keys_out;
  uint64_t* lst;
  int c_slots;                // chunk slots of the centroid rows (fixes the list shape)
  uint64_t* part;
  const int32_t* c2t;
  const void* tiles;
  const uint16_t* scales;
  int32_t* probe_out;
  float* logits_out;
  int32_t* tokens_out;
  int32_t* token;
};
// fh_b1.hip, one object per row format: stage 1 by the centroids' format, selection + stage 2
// (+ token) by the tiles' format.
hipError_t launch_b1_scores_f32(const B1Args& a, hipStream_t st);
hipError_t launch_b1_scores_bf16(const B1Args& a, hipStream_t st);
hipError_t launch_b1_scores_int4(const B1Args& a, hipStream_t st);
hipError_t launch_b1_stage2_f32(const B1Args& a, hipStream_t st);
hipError_t launch_b1_stage2_bf16(const B1Args& a, hipStream_t st);
hipError_t launch_b1_stage2_int4(const B1Args& a, hipStream_t st);
// B = 1 probe selection fused with stage 2 (one kernel, then the token decode); reads the
// keys launch_scores left in the workspace.
hipError_t launch_stage2_b1(const HeadShape& s, int p, const void* h, const int32_t* c2t, const void* tiles,
                            const uint16_t* scales, const Sampling& smp, const Workspace& ws, int32_t* probe_out,
                            float* logits_out, int32_t* tokens_out, int32_t* token, hipStream_t st);
hipError_t launch_dense(const HeadShape& s, int V, const void* h, const void* E, const Sampling& smp,
                        uint64_t* best, int32_t* token, float* logits, hipStream_t st);
hipError_t launch_centroids(int d, int c, int b, int src_bf16, int dst_bf16, int unit, const void* E,
                            const int32_t* c2t, void* out, hipStream_t st);
// Monte-Carlo marginal (fh_mc.hip): the forward workspace for p = c, then the centroid
// logits s (and s / tau, prefilter thresholds), all token logits z (tile order), the per-cluster softmax statistics M and Zc,
// the accumulated weights A, the per-row minimum cell and the forward's token output.
struct McWorkspace {
  Workspace fw;
  float* s;           // [B][c]
  float* stau;        // [B][c] s / tau
  uint32_t* t0u;      // [B] prefilter thresholds
  float* range;       // [B][2] key range
  float* mu;          // [B][256] expected key counts above candidate thresholds
  float* z;           // [B][c][b]
  double* M;          // [B][c]
  double* Zc;         // [B][c]
  double* A;          // [B][c]
  uint64_t* minneg;   // [B]
  int32_t* token;     // [B]
  size_t bytes;
};
McWorkspace carve_mc_workspace(void* base, int B, int c, int b);
// Reads w.s and w.z (written by the forward path) and writes out[B][V].
hipError_t launch_mc(const HeadShape& s, int p, float tau, uint64_t seed, int64_t n_sets, int clip,
                     const int32_t* c2t, const McWorkspace& w, double* out, hipStream_t st);
// Offline balanced spherical k-means (fh_cluster.hip); synchronises `st` once per round.
size_t build_clusters_workspace_bytes(int V, int d, int c);
hipError_t launch_build_clusters(int V, int d, int c, int src_bf16, const void* E, int iters, uint64_t seed, int unit,
                                 int dst_bf16, void* centroids, int32_t* c2t, void* ws, hipStream_t st);
// int4 rows ([rows][d/2] nibbles) followed by their bf16 group scales ([rows][d/128]) in one
// buffer: the scales start at this byte offset.
inline size_t int4_scales_offset(size_t rows, size_t d) { return (rows * d / 2 + 255) & ~(size_t)255; }
inline size_t int4_rows_bytes(size_t rows, size_t d) { return int4_scales_offset(rows, d) + rows * (d / 128) * 2; }
hipError_t launch_quant_int4_rows(const uint16_t* src, int rows, int d, uint8_t* q, uint16_t* scales,
                                  hipStream_t st);
// The sampler's Philox words / fp32 Gumbel values for elements n0 .. n0 + count - 1 (fh_util.hip).
hipError_t launch_philox_words(uint64_t seed, uint32_t row, uint64_t step, uint32_t stream, uint32_t n0,
                               int64_t count, uint32_t* words, float* gum, hipStream_t st);
// B > 1: clears the selection's per-cluster state (row masks, kept flags, kept count).
hipError_t launch_clear_select(const Workspace& ws, int c, hipStream_t st);
hipError_t launch_pack(int V, int d, int c, int b, int src_bf16, int dst_fmt, const void* E,
                       const int32_t* c2t, void* tiles, uint16_t* scales, uint32_t* counts,
                       uint32_t* bad, hipStream_t st);

}  // namespace fh
