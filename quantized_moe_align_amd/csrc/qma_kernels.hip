// HIP kernels of libqma for gfx950 (CDNA4): block-aligned routing
// (moe_align), weight prepack, the W4A16 expert GEMMs, the split-K
// reduction, the SiLU-gated activation, the top-k combine and the router's
// top-k softmax.
//
// The passages followed are cited per kernel (page titles in include/qma.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "qma_internal.h"

namespace qma {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// moe_align: stable counting sort of routed slots by expert, each expert
// padded to a multiple of the block size ([announce] scheduling section; the
// buffers may be over-allocated: [release] runtime considerations).
//
// One workgroup of 8 waves. Wave w owns a contiguous range of slots. Pass 1
// counts slots per (wave, expert) in LDS. A scan turns the counts into
// per-(wave, expert) start positions that follow expert order, then wave
// order, so positions ascend with the slot index. Pass 2 walks each wave's
// range in 64-slot steps. A lane's rank among the lanes holding the same
// expert comes from ballots over the expert id's bits, which keeps the
// within-step order by lane. The result is deterministic and needs no
// global atomics.
// ---------------------------------------------------------------------------
constexpr int kAlignWaves = 8;
constexpr int kAlignThreads = kAlignWaves * 64;
constexpr int kAlignUnroll = 8;   // ids each lane loads before using any

__global__ __launch_bounds__(kAlignThreads) void moe_align_kernel(
    const int32_t* __restrict__ ids, int32_t R, int32_t E, int32_t B,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ ntp_out, int32_t cap, int32_t blocks_cap) {
  extern __shared__ int32_t smem[];
  int32_t* wc = smem;                       // [waves][E]
  int32_t* cnt = wc + kAlignWaves * E;      // [E]
  int32_t* off = cnt + E;                   // [E + 1]
  int32_t* wsum = off + E + 1;              // [waves]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) wc[i] = 0;
  __syncthreads();
  const int per = (R + kAlignWaves - 1) / kAlignWaves;
  const int lo = min(R, w * per), hi = min(R, lo + per);
  // the ids of kAlignUnroll rows of 64 slots are loaded together, so a
  // wave waits out one memory round trip per batch rather than per row
  constexpr int U = kAlignUnroll;
  for (int base = lo; base < hi; base += 64 * U) {
    int ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * 64 + lane;
      ev[u] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if ((unsigned)ev[u] < (unsigned)E) atomicAdd(&wc[w * E + ev[u]], 1);
  }
  __syncthreads();
  // per expert: total, and exclusive prefix over waves (in place)
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = 0;
    for (int v = 0; v < kAlignWaves; ++v) {
      const int c = wc[v * E + e];
      wc[v * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  // exclusive scan of padded counts over experts; each thread takes a
  // contiguous run of experts (E <= 1024 -> at most 2 per thread)
  const int ept = (E + kAlignThreads - 1) / kAlignThreads;
  const int e0 = min(E, tid * ept), e1 = min(E, e0 + ept);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += (cnt[e] + B - 1) / B * B;
  int incl = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int v = 0; v < w; ++v) wave_base += wsum[v];
  int run = wave_base + incl - local;
  for (int e = e0; e < e1; ++e) {
    off[e] = run;
    run += (cnt[e] + B - 1) / B * B;
  }
  if (tid == kAlignThreads - 1) off[E] = run;
  __syncthreads();
  const int ntp = off[E];
  if (tid == 0) *ntp_out = ntp;
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) wc[i] += off[i % E];
  // expert of each block (binary search in the offsets), -1 past the end
  for (int b = tid; b < blocks_cap; b += kAlignThreads) {
    const int p = b * B;
    int e = -1;
    if (p < ntp) {
      int l = 0, h = E - 1;  // largest e with off[e] <= p
      while (l < h) {
        const int m = (l + h + 1) >> 1;
        if (off[m] <= p) l = m; else h = m - 1;
      }
      e = l;
    }
    expert_ids[b] = e;
  }
  // sentinel padding inside each expert's segment, and the tail
  // (large blocks: one wave per expert, its lanes over the up to B - 1
  // padding positions; small blocks: one thread per expert)
  if (B >= 64) {
    for (int e = w; e < E; e += kAlignWaves)
      for (int p = off[e] + cnt[e] + lane; p < off[e + 1]; p += 64) sorted_ids[p] = R;
  } else {
    for (int e = tid; e < E; e += kAlignThreads)
      for (int p = off[e] + cnt[e]; p < off[e + 1]; ++p) sorted_ids[p] = R;
  }
  for (int p = ntp + tid; p < cap; p += kAlignThreads) sorted_ids[p] = R;
  __syncthreads();
  // pass 2: place each slot; lanes of a row holding the same expert are
  // found with one ballot per bit of the expert index
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 1;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base0 = lo; base0 < hi; base0 += 64 * U) {
    int ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base0 + u * 64 + lane;
      ev[u] = i < hi ? ids[i] : -1;
    }
    // rows in slot order, so each expert's slots stay ascending
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = base0 + u * 64;
      if (base >= hi) break;
      const int i = base + lane;
      const int e = ev[u];
      const bool valid = (unsigned)e < (unsigned)E;
      uint64_t peers = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = valid && ((e >> bit) & 1);
        const uint64_t m = __ballot(set);
        peers &= set ? m : ~m;
      }
      const int rank = __popcll(peers & below);
      int pos = 0;
      if (valid) pos = wc[w * E + e];
      if (valid) sorted_ids[pos + rank] = i;
      if (valid && (peers & below) == 0) wc[w * E + e] = pos + __popcll(peers);
    }
  }
}

int launch_moe_align(const int32_t* ids, int32_t R, int32_t E, int32_t B,
                     int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                     int32_t cap, void* stream) {
  const int32_t blocks_cap = (cap + B - 1) / B;
  const size_t lds = sizeof(int32_t) * ((size_t)kAlignWaves * E + E + E + 1 + kAlignWaves);
  hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(kAlignThreads), lds,
                     (hipStream_t)stream, ids, R, E, B, sorted_ids, expert_ids, ntp, cap,
                     blocks_cap);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// prepack: checkpoint layout -> MFMA-fragment-ordered 128-wide K chunks
// (layout fixed at load: [announce] scheduling section; BLOCK_K = 128
// packing: [release] grouped techniques). See qma_internal.h for the layout.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t interleave_nibbles(uint32_t w) {
  // out nibble p <- in nibble {0,4,1,5,2,6,3,7}[p]: the even nibbles then
  // hold k0..k3 and the odd nibbles k4..k7, so one mask (and one shift)
  // spreads them over bytes in k order.
  uint32_t r = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int src = (p & 1) ? 4 + (p >> 1) : (p >> 1);
    r |= ((w >> (4 * src)) & 0xFu) << (4 * p);
  }
  return r;
}

// Output block number b (of 1 KiB weights or 128-byte scales) -> expert,
// tile and K chunk, in the block order of the packed layout.
__device__ __forceinline__ void block_place(int64_t b, int64_t n_tiles, int64_t k_chunks,
                                            int wg_log2, int64_t& e, int64_t& nt, int64_t& kc) {
  const int64_t g = (int64_t)1 << wg_log2;
  const int64_t r = b & (g - 1);
  int64_t rest = b >> wg_log2;
  kc = rest % k_chunks;
  rest /= k_chunks;
  const int64_t groups = n_tiles >> wg_log2;
  nt = (rest % groups) * g + r;
  e = rest / groups;
}

// Packed tile nt -> checkpoint tile. A gate_up layer with the activation
// fused keeps gate tile q and up tile q side by side (packed 2q, 2q + 1).
__device__ __forceinline__ int64_t source_tile(int64_t nt, int64_t n_tiles, int32_t act) {
  if (!act) return nt;
  return (nt & 1) ? n_tiles / 2 + (nt >> 1) : (nt >> 1);
}

__global__ void prepack_weights_kernel(const uint32_t* __restrict__ qw, uint32_t* __restrict__ out,
                                       int32_t N, int32_t K, int64_t n_tiles, int64_t k_chunks,
                                       int32_t wg_log2, int32_t act, int64_t total) {
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(o & 3);
    const int l = (int)((o >> 2) & 63);
    int64_t e, nt, kc;
    block_place(o >> 8, n_tiles, k_chunks, wg_log2, e, nt, kc);
    const int64_t n = source_tile(nt, n_tiles, act) * 16 + (l & 15);
    const int64_t k0 = kc * 128 + j * 32 + (l >> 4) * 8;
    out[o] = interleave_nibbles(qw[(e * N + n) * (K / 8) + k0 / 8]);
  }
}

__global__ void prepack_scales_kernel(const uint16_t* __restrict__ sc, uint16_t* __restrict__ out,
                                      int32_t N, int32_t K, int64_t n_tiles, int64_t k_chunks,
                                      int32_t wg_log2, int32_t act, int64_t total) {
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(o & 3);
    const int row = (int)((o >> 2) & 15);
    int64_t e, nt, kc;
    block_place(o >> 6, n_tiles, k_chunks, wg_log2, e, nt, kc);
    const int64_t n = source_tile(nt, n_tiles, act) * 16 + row;
    out[o] = sc[(e * N + n) * (K / 32) + kc * 4 + g];
  }
}

int launch_prepack(const Layer& L, const int32_t* qweight, const uint16_t* scales,
                   void* packed, void* stream) {
  const int64_t words = (int64_t)(L.w_bytes / 4);
  const int64_t svals = (int64_t)(L.s_bytes / 2);
  auto blocks = [](int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); };
  hipLaunchKernelGGL(prepack_weights_kernel, dim3(blocks(words)), dim3(256), 0,
                     (hipStream_t)stream, (const uint32_t*)qweight, (uint32_t*)packed, L.N, L.K,
                     L.n_tiles, L.k_chunks, L.wg_log2, L.act, words);
  hipLaunchKernelGGL(prepack_scales_kernel, dim3(blocks(svals)), dim3(256), 0,
                     (hipStream_t)stream, scales, (uint16_t*)((char*)packed + L.w_bytes), L.N,
                     L.K, L.n_tiles, L.k_chunks, L.wg_log2, L.act, svals);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small-M expert GEMM (decode shapes: 16 to 64 rows per tile).
//
// One v_mfma_f32_16x16x32_bf16 takes 16 tokens as its rows and 16 weight
// rows (output columns) as its columns, and covers exactly one 32-wide
// scale group. Each lane then owns one output column and needs one scale
// per group. Both MFMA dimensions are 16 on CDNA4, so a handful of tokens
// per expert fills the matrix core without exchanging operand roles. (The
// pages' decode kernel puts weights on the MMA M side because its MMA is
// 16x8: [announce] scheduling section.)
//
// The weight operand is the exact bf16 value 128+q, made from the nibbles
// by an and-or, so dequantisation never rounds. The zero point enters
// through the accumulator input: an MFMA against a constant -136 operand
// gives -136 * sum_k x_k, so each MFMA yields sum_k x_k (q_k - 8), and the
// group's scale is applied in fp32:
//     acc += scale[n, g] * ( sum_k x_k (128 + q_k) - 136 sum_k x_k ).
//
// Workgroup: 4 waves. WK of them split the workgroup's K range and 4/WK
// split its columns. A wave owns NTW 16-column weight tiles and TM 16-token
// tiles. It streams its weights with buffer loads: per 128-wide K chunk, a
// 1 KiB contiguous block per tile, with D chunks in flight. Token rows are
// gathered with buffer loads whose out-of-range offset returns zeros for
// rows the tile does not use, so those rows are never read. The WK partial
// sums meet in LDS at the end.
// ---------------------------------------------------------------------------
// silu(g) * u in fp32 (the activation of the gated MLP between gate_up and
// down: [announce] measurement section).
__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) = g * sigmoid(g), without a branch. With h = e^(-|g|/2) (never
  // overflows) and e^(-|g|) = h h: sigmoid(g) = 1 / (1 + h h) for g >= 0 and
  // h h / (1 + h h) for g < 0, so silu(g) = ((g a) a) / (1 + h h) with a = 1
  // or h. Multiplying by a twice keeps g e^g a normal number wherever it is
  // one (e^g alone underflows below -87.3). The divisor lies in [1, 2],
  // where the hardware reciprocal (1 ulp) replaces the correctly rounded
  // division's scaling steps; the fp32 result stays far inside one bf16 ulp
  // of the exact value.
  const float h = __expf(-0.5f * __builtin_fabsf(g));
  const float a = g >= 0.0f ? 1.0f : h;
  return ((g * a) * a) * __builtin_amdgcn_rcpf(1.0f + h * h) * u;
}

// One output of a gate_up GEMM with the activation fused: the gate and up
// sums are each rounded to bf16 first, as the unfused GEMM stores them, so
// the result equals the activation kernel applied to the unfused output.
__device__ __forceinline__ uint16_t fused_silu_mul(float g, float u) {
  const float gb = __uint_as_float(pack_bf16x2(g, 0.f) << 16);
  const float ub = __uint_as_float(pack_bf16x2(u, 0.f) << 16);
  return (uint16_t)(pack_bf16x2(silu_mul(gb, ub), 0.f) & 0xFFFFu);
}

struct GemmParams {
  const uint16_t* a;
  const uint8_t* wpk;
  const uint8_t* spk;
  uint16_t* c;
  float* ws;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntp;
  const float* topk_w;
  const int32_t* m_indices;
  const int32_t* masked_m;
  uint32_t a_bytes;
  int32_t mode, a_row_div, num_tiles, nblocks, split, num_slots;
  int32_t Mb, tiles_per_expert, rows_cap, cap;
  int32_t E, N, K, NT, KC, BM;
  int32_t nstream, nbtot;  // streaming small-M: N blocks per workgroup, N blocks in all
  int32_t* work;            // dynamic schedule: work counter (workspace)
  int32_t wg_log2;          // packed layout: log2 of the tiles per block group
  int32_t fold;             // column-block groups per tile dealt to the XCDs (divides nblocks)
  int32_t act;              // 1: gate_up with silu(gate) * up fused; output row stride N / 2
};

// Place of 16-column tile t0 + j, K chunk c inside one expert's packed
// weights or scales (unit = the block size, kWBlockBytes or kSBlockBytes):
// byte offset base + j * tile + c * chunk, for j within t0's tile group
// (callers keep a wave's tiles inside one group: group sizes are 1 or 16,
// and each wave's first tile is a multiple of its tile count).
struct TileAddr {
  uint32_t base, tile, chunk;
};
__device__ __forceinline__ TileAddr tile_addr(const GemmParams& p, int t0, uint32_t unit) {
  const int lg = p.wg_log2;
  const uint32_t g = 1u << lg;
  const uint32_t grp = (uint32_t)t0 >> lg, r = (uint32_t)t0 & (g - 1);
  return {(grp * (uint32_t)p.KC * g + r) * unit, (lg ? 1u : (uint32_t)p.KC) * unit, g * unit};
}

struct RowInfo {
  bool valid;
  int32_t a_row;
  int32_t out_row;
};

// The tile's expert, or -1 for a tile with no work. (tile < num_tiles, so
// expert_ids[tile] lies inside the buffer even past the routed blocks; it is
// read beside num_tokens_padded rather than after it, one memory round trip
// instead of two.)
__device__ __forceinline__ int tile_expert(const GemmParams& p, int tile) {
  if (p.mode == 0) {
    const int ntp = *p.ntp;
    const int e = p.expert_ids[tile];
    return (tile * p.BM < ntp && e >= 0 && e < p.E) ? e : -1;
  }
  if (p.mode == 1) {
    const int e = p.m_indices[tile * p.BM];
    return (e >= 0 && e < p.E) ? e : -1;
  }
  // masked: tiles are numbered row-block-major (tile = jt * E + e), so the
  // tiles that hold rows come first and spread evenly over the XCDs
  const int e = tile % p.E;
  const int jt = tile / p.E;
  const int mm = min(max(p.masked_m[e], 0), p.Mb);
  return (jt * p.BM < mm) ? e : -1;
}

// Row r of a tile: whether it holds a token, its activation row and its
// output row. A tile without an expert (e < 0) holds none, and nothing is
// read for it: a masked layer would otherwise index masked_m[-1].
__device__ __forceinline__ RowInfo row_info(const GemmParams& p, int tile, int e, int r) {
  RowInfo ri{false, 0, 0};
  if (e < 0) return ri;
  if (p.mode == 0) {
    const int pos = tile * p.BM + r;
    const int s = (pos < p.cap) ? p.sorted_ids[pos] : -1;
    if (s >= 0 && s < p.num_slots) {
      ri.valid = true;
      ri.a_row = s / p.a_row_div;
      ri.out_row = s;
    }
  } else if (p.mode == 1) {
    const int row = tile * p.BM + r;
    if (p.m_indices[row] == e) {
      ri.valid = true;
      ri.a_row = row;
      ri.out_row = row;
    }
  } else {
    const int jt = tile / p.E;
    const int mm = min(max(p.masked_m[e], 0), p.Mb);
    const int rr = jt * p.BM + r;
    if (rr < mm) {
      ri.valid = true;
      ri.a_row = e * p.Mb + rr;
      ri.out_row = ri.a_row;
    }
  }
  return ri;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// bytes 2H, 2H+1 of v (each 0..15) -> two exact floats
template <bool H>
__device__ __forceinline__ f32x2 byte_pair(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 512.0f, H);
}

// One packed word (k0 k4 k1 k5 k2 k6 k3 k7) -> bf16((q - 8) s) for k0..k7
// in order: two nibbles at a time become exact floats (a byte holding q in
// 0..15, read as an OCP e4m3 code with power-of-two scale 512, is exactly q),
// then q s - 8 s is one fp32 FMA, rounded once to bf16. About 19 VALU per
// word, whatever the number of token rows that share it.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s, float neg8s) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // bytes k0 k1 k2 k3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // bytes k4 k5 k6 k7
  const f32x2 q01 = byte_pair<false>(lo), q23 = byte_pair<true>(lo);
  const f32x2 q45 = byte_pair<false>(hi), q67 = byte_pair<true>(hi);
  return u32x4{cvt_pk_bf16(__builtin_fmaf(q01.x, s, neg8s), __builtin_fmaf(q01.y, s, neg8s)),
               cvt_pk_bf16(__builtin_fmaf(q23.x, s, neg8s), __builtin_fmaf(q23.y, s, neg8s)),
               cvt_pk_bf16(__builtin_fmaf(q45.x, s, neg8s), __builtin_fmaf(q45.y, s, neg8s)),
               cvt_pk_bf16(__builtin_fmaf(q67.x, s, neg8s), __builtin_fmaf(q67.y, s, neg8s))};
}


// One packed word -> the eight exact bf16 values 128 + q, in k order: the
// bf16 pattern 0x43qq is 128 + q, so each output word is two value bytes
// interleaved with the constant 0x43 (v_perm_b32 byte selects).
__device__ __forceinline__ u32x4 unpack_128q(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // bytes k0 k1 k2 k3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // bytes k4 k5 k6 k7
  u32x4 r;
  r.x = __builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u);
  r.y = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u);
  r.z = __builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u);
  r.w = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u);
  return r;
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int kBufWord3 = 0x00020000;  // raw 32-bit buffer resource, gfx9 family
constexpr int kNonTemporal = 2;        // streaming load: weights are read once

// A pointer the compiler may not prove wave-uniform, made so (every lane
// holds the same value): a buffer resource built from it then stays in
// scalar registers instead of needing a loop over lanes per load.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufWord3);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Reads of LDS filled by direct-to-LDS loads are issued as ds_read_b128 in
// inline asm and waited with explicit counts (wait_lgkm ties the wait to the
// register it guards, so the consumer cannot move above it). The compiler
// then tracks no such read: its own wait counts for direct-to-LDS loads turn
// conservative where control flow merges and would wait for every
// prefetch. LDS operations complete in order, so these reads can only make
// the compiler's own counts stricter.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
  return v;
}

// Bare workgroup barrier. __syncthreads() also fences memory, and that
// fence waits for every outstanding direct-to-LDS load, including prefetches
// of later chunks. The kernels that use this wait with explicit vmcnt
// counts, and the asm clobbers keep the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_lgkm(u32x4& v) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}

// Decode the XCD-aware workgroup order. Workgroup i runs on XCD i % 8. The
// column blocks of a token tile form p.fold groups, each a virtual tile
// (tile * fold + group), and XCD x takes virtual tiles x, x+8, ... with all
// of their (column block, split) pieces. A tile's activations then stay in
// the L2 of the XCDs that hold its groups (one without folding), and empty
// tiles spread evenly over the XCDs.
__device__ __forceinline__ bool decode_bid(const GemmParams& p, int bid, int& tile, int& nb,
                                           int& sp) {
  const int xcd = bid & 7;
  const int idx = bid >> 3;
  const int nbf = p.nblocks / p.fold;
  const int per_vt = nbf * p.split;
  const int j = idx / per_vt;
  const int rem = idx - j * per_vt;
  const int vt = xcd + 8 * j;
  tile = vt / p.fold;
  nb = (vt - tile * p.fold) * nbf + rem / p.split;
  sp = rem % p.split;
  return tile < p.num_tiles;
}

// Workgroup order of the large-M kernel. Workgroup i runs on XCD i % 8.
// The routed tiles are dealt to the XCDs in turn (XCD x takes tiles x,
// x + 8, ...), each with all of its (column block, split) pieces, which run
// together so that the tile's token rows stay in that XCD's L2. Dealing in
// turn spreads a large expert's full tiles, and the partly filled tiles that
// end each expert's rows, evenly over the XCDs; contiguous ranges of the
// tile list would put a large expert's tiles on one or two XCDs, which then
// set the launch time. The routed tile count is read on the device.
__device__ __forceinline__ bool decode_bid_lm(const GemmParams& p, int& tile, int& nb, int& sp) {
  const int ntiles = p.mode == 0 ? min(*p.ntp / p.BM, p.num_tiles) : p.num_tiles;
  const int per = p.nblocks * p.split;
  const int bid = blockIdx.x;
  const int j = bid >> 3;
  const int s = j / per;
  tile = (bid & 7) + 8 * s;
  if (tile >= ntiles) return false;
  const int nbsp = j - s * per;
  nb = nbsp / p.split;
  sp = nbsp - nb * p.split;
  return true;
}

template <int TM, int NTW, int WK, int D>
__global__ __launch_bounds__(256, 2) void gemm_small_m_kernel(const GemmParams p) {
  constexpr int WN = 4 / WK;
  constexpr int NACC = NTW * TM * 4;
  __shared__ float s_red[WK > 1 ? 4 * NACC * 64 : 1];

  int tile, nb, sp;
  if (!decode_bid(p, blockIdx.x, tile, nb, sp)) return;
  const int e = __builtin_amdgcn_readfirstlane(tile_expert(p, tile));
  if (e < 0) return;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wk = w % WK, wn = w / WK;
  const int col = lane & 15, kb = lane >> 4;

  const int cs0 = (int)(((int64_t)sp * p.KC) / p.split);
  const int cs1 = (int)(((int64_t)(sp + 1) * p.KC) / p.split);
  const int c_begin = cs0 + ((cs1 - cs0) * wk) / WK;
  const int c_end = cs0 + ((cs1 - cs0) * (wk + 1)) / WK;

  const int nt0 = (nb * WN + wn) * NTW;  // first 16-column tile of this wave
  const uint32_t tile_bytes = (uint32_t)p.KC * kWBlockBytes;
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(p.wpk + (size_t)e * p.NT * tile_bytes, (uint32_t)p.NT * tile_bytes);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(p.spk + (size_t)e * p.NT * p.KC * kSBlockBytes,
                (uint32_t)p.NT * p.KC * kSBlockBytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
  const TileAddr wa = tile_addr(p, nt0, kWBlockBytes), sa = tile_addr(p, nt0, kSBlockBytes);
  const uint32_t voff_w = lane * 16 + wa.base;
  const uint32_t voff_s = col * 8 + sa.base;
  uint32_t voff_x[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const RowInfo ri = row_info(p, tile, e, tm * 16 + col);
    voff_x[tm] = ri.valid ? (uint32_t)ri.a_row * (uint32_t)p.K * 2u + kb * 16 : 0x80000000u;
  }

  struct Stage {
    u32x4 w[NTW];
    u32x2 s[NTW];
    u32x4 x[TM][4];
  };
  Stage st[D];

  auto load = [&](Stage& s, int c) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      s.w[nt] = __builtin_amdgcn_raw_buffer_load_b128(rw, voff_w, nt * wa.tile + c * wa.chunk,
                                                      kNonTemporal);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      s.s[nt] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff_s, nt * sa.tile + c * sa.chunk, 0);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        s.x[tm][g] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff_x[tm] + g * 64, c * 256, 0);
  };

  f32x4 acc[NTW][TM];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) acc[nt][tm] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 neg136 = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage& s) {
    if constexpr (TM == 1 && NTW == 4) {
      // zero-point MFMAs first, then products one (group, column tile)
      // pair ahead of their scale FMAs (same per-accumulator order as the
      // loop below), so no MFMA result is read right after its issue
      f32x4 xs[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) xs[g] = mfma16(s.x[0][g], neg136, zero4);
      f32x4 pr[2];
      float scv[2];
      auto product = [&](int i) {
        const int g = i / NTW, nt = i % NTW;
        const u32x4 wb = unpack_128q(s.w[nt][g]);
        const uint32_t sw = s.s[nt][g >> 1];
        scv[i & 1] = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
        pr[i & 1] = mfma16(s.x[0][g], wb, xs[g]);
      };
      auto scale = [&](int i) {
        const int nt = i % NTW;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[nt][0][r] = __builtin_fmaf(scv[i & 1], pr[i & 1][r], acc[nt][0][r]);
      };
      product(0);
#pragma unroll
      for (int i = 1; i < 4 * NTW; ++i) {
        product(i);
        scale(i - 1);
      }
      scale(4 * NTW - 1);
      return;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (NTW == 1) {
        // one column tile: each row tile's zero-point sum is used once, so
        // it is formed just before its product (same operations and order)
        const u32x4 wb = unpack_128q(s.w[0][g]);
        const uint32_t sw = s.s[0][g >> 1];
        const float scv = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const f32x4 pr = mfma16(s.x[tm][g], wb, mfma16(s.x[tm][g], neg136, zero4));
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[0][tm][r] = __builtin_fmaf(scv, pr[r], acc[0][tm][r]);
        }
        continue;
      }
      f32x4 xs[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) xs[tm] = mfma16(s.x[tm][g], neg136, zero4);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const uint32_t wq = s.w[nt][g];
        const u32x4 wb = unpack_128q(wq);
        const uint32_t sw = s.s[nt][g >> 1];
        const float scv = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const f32x4 pr = mfma16(s.x[tm][g], wb, xs[tm]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nt][tm][r] = __builtin_fmaf(scv, pr[r], acc[nt][tm][r]);
        }
      }
    }
  };

  // K loop with D chunks in flight. Waves with at least 2*D chunks run a
  // main loop whose loads are unconditional, so the wait counts before each
  // use allow every later chunk's loads to stay in flight; only the final
  // drain (and short ranges) take the guarded path.
  int c = c_begin;
  if (c_end - c_begin >= 2 * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      __builtin_amdgcn_sched_barrier(0);
      load(st[d], c + d);
    }
    for (; c + 2 * D <= c_end; c += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        // The barriers keep each stage's loads in issue order behind its
        // compute; without them the scheduler sinks loads of one stage past
        // the next stage's compute and the wait counts serialise the stages.
        __builtin_amdgcn_sched_barrier(0);
        compute(st[d]);
        __builtin_amdgcn_sched_barrier(0);
        load(st[d], c + D + d);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (c + d < c_end) load(st[d], c + d);
  }
  for (; c < c_end; c += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (c + d < c_end) {
        compute(st[d]);
        if (c + d + D < c_end) load(st[d], c + d + D);
      }
    }
  }

  // Output: lane holds rows (tokens) tm*16 + 4*kb + r of column col.
  auto store = [&](int nt, int tm, int r, float v) {
    const RowInfo ri = row_info(p, tile, e, tm * 16 + kb * 4 + r);
    if (!ri.valid) return;
    const int n = (nt0 + nt) * 16 + col;
    if (p.split > 1) {
      p.ws[((size_t)sp * p.rows_cap + ri.out_row) * p.N + n] = v;
    } else {
      const float t = (p.mode == 0 && p.topk_w) ? p.topk_w[ri.out_row] : 1.0f;
      p.c[(size_t)ri.out_row * p.N + n] = (uint16_t)(pack_bf16x2(v * t, 0.f) & 0xFFFFu);
    }
  };
  // fused activation: tiles nt (gate) and nt + 1 (up) of a pair
  auto store_pair = [&](int nt, int tm, int r, float g, float u) {
    const RowInfo ri = row_info(p, tile, e, tm * 16 + kb * 4 + r);
    if (!ri.valid) return;
    const float t = (p.mode == 0 && p.topk_w) ? p.topk_w[ri.out_row] : 1.0f;
    p.c[(size_t)ri.out_row * (p.N / 2) + ((nt0 + nt) / 2) * 16 + col] =
        fused_silu_mul(g * t, u * t);
  };
  const bool fused = p.act && p.split == 1;

  if constexpr (WK == 1) {
    if (fused) {
      if constexpr (NTW % 2 == 0) {
#pragma unroll
        for (int nt = 0; nt < NTW; nt += 2)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int r = 0; r < 4; ++r) store_pair(nt, tm, r, acc[nt][tm][r], acc[nt + 1][tm][r]);
      }
      return;
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 4; ++r) store(nt, tm, r, acc[nt][tm][r]);
  } else {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_red[(w * NACC + (nt * TM + tm) * 4 + r) * 64 + lane] = acc[nt][tm][r];
    __syncthreads();
    if (fused) {
      // wave (wk, wn) finishes tile pairs wk, wk + WK, ... of its group
      if constexpr (NTW % 2 == 0) {
        for (int pr = wk; pr < NTW / 2; pr += WK) {
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int ig = (2 * pr * TM + tm) * 4 + r, iu = ((2 * pr + 1) * TM + tm) * 4 + r;
              float g = 0.f, u = 0.f;
#pragma unroll
              for (int j = 0; j < WK; ++j) {
                g += s_red[((wn * WK + j) * NACC + ig) * 64 + lane];
                u += s_red[((wn * WK + j) * NACC + iu) * 64 + lane];
              }
              store_pair(2 * pr, tm, r, g, u);
            }
        }
      }
      return;
    }
    // wave (wk, wn) finishes tiles nt = wk, wk + WK, ... of its column group
    for (int nt = wk; nt < NTW; nt += WK) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = (nt * TM + tm) * 4 + r;
          float v = 0.f;
#pragma unroll
          for (int j = 0; j < WK; ++j) v += s_red[((wn * WK + j) * NACC + i) * 64 + lane];
          store(nt, tm, r, v);
        }
    }
  }
}

// Streaming small-M variant for short K: one 16-token tile, one K
// partition, the four waves side by side over 16 * NTW columns each. A
// workgroup walks p.nstream consecutive column blocks of its expert: the
// (column block, K chunk) pairs form one stream through the D-stage load
// pipeline, so the next block's weights are in flight while the current
// block finishes, and a block's outputs are stored as soon as its last
// chunk is accumulated. Token rows, output rows and topk weights are looked
// up once per workgroup. With XR (K of one or two chunks) the token rows
// are loaded once and stay in registers; the stages then hold weights
// only, and two of them leave room for three workgroups per CU (TP8 down
// share: 89.1-89.4 -> 81.9-82.2 us against four stages with the rows in
// every stage; 83.1-83.8 us with resident rows and four stages at two
// workgroups per CU).
template <int NTW, int D, bool XR>
__global__ __launch_bounds__(256, XR ? 3 : 2) void gemm_small_m_stream_kernel(const GemmParams p) {
  static_assert(!XR || D % 2 == 0, "resident token rows: stage d holds chunk d % 2");
  int tile, grp, sp;
  if (!decode_bid(p, blockIdx.x, tile, grp, sp)) return;
  const int e = __builtin_amdgcn_readfirstlane(tile_expert(p, tile));
  if (e < 0) return;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int col = lane & 15, kb = lane >> 4;
  const int KC = p.KC;
  const int nb0 = grp * p.nstream;
  const int total = min(p.nstream, p.nbtot - nb0) * KC;

  // Weights of the whole expert; this wave's tiles of column block nb are
  // (nb * 4 + w) * NTW + nt.
  const uint32_t tile_bytes = (uint32_t)KC * kWBlockBytes;
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(p.wpk + (size_t)e * p.NT * tile_bytes, (uint32_t)p.NT * tile_bytes);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(p.spk + (size_t)e * p.NT * KC * kSBlockBytes, (uint32_t)p.NT * KC * kSBlockBytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
  const uint32_t voff_w = lane * 16;
  const uint32_t voff_s = col * 8;
  const RowInfo rx = row_info(p, tile, e, col);
  const uint32_t voff_x = rx.valid ? (uint32_t)rx.a_row * (uint32_t)p.K * 2u + kb * 16 : 0x80000000u;
  int32_t out_row[4];
  float tw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const RowInfo ri = row_info(p, tile, e, kb * 4 + r);
    out_row[r] = ri.valid ? ri.out_row : -1;
    tw[r] = (ri.valid && p.mode == 0 && p.topk_w) ? p.topk_w[ri.out_row] : 1.0f;
  }

  struct Stage {
    u32x4 w[NTW];
    u32x2 s[NTW];
    u32x4 x[XR ? 1 : 4];
  };
  Stage st[D];
  // K of one or two chunks (XR): the tile's token rows for both chunks stay
  // in registers for the whole stream instead of riding in every stage;
  // the stream starts on chunk 0 and D is even, so stage d always holds
  // chunk d % 2 (a one-chunk K loads chunk 0 twice).
  u32x4 xres[XR ? 2 : 1][4];
  if constexpr (XR) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        xres[c][g] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff_x + g * 64,
                                                           min(c, KC - 1) * 256, 0);
  }
  // load cursor: column block and chunk of the next stage to fetch
  int l_nb = nb0, l_c = 0;
  auto load_next = [&](Stage& s) {
    // this wave's tiles of column block l_nb: (l_nb * 4 + w) * NTW + nt
    const int t0 = (l_nb * 4 + w) * NTW;
    const TileAddr wa = tile_addr(p, t0, kWBlockBytes), sa = tile_addr(p, t0, kSBlockBytes);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      s.w[nt] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, voff_w, wa.base + nt * wa.tile + l_c * wa.chunk, kNonTemporal);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      s.s[nt] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff_s,
                                                     sa.base + nt * sa.tile + l_c * sa.chunk, 0);
    if constexpr (!XR) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        s.x[g] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff_x + g * 64, l_c * 256, 0);
    }
    if (++l_c == KC) {
      l_c = 0;
      ++l_nb;
    }
  };

  f32x4 acc[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 neg136 = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // compute cursor: column block and chunk of the next stage to consume
  int c_nb = nb0, c_c = 0;
  auto step = [&](const Stage& s, int d) {
    const u32x4* sx;
    if constexpr (XR)
      sx = xres[d & 1];
    else
      sx = s.x;
    if constexpr (NTW == 4) {
      // The four zero-point MFMAs go first and products run one (group,
      // column tile) pair ahead of their scale FMAs, so no MFMA result is
      // read right after its issue; each accumulator takes the same
      // operations in the same order as the plain loop below. (With two
      // column tiles the extra registers would cost a workgroup per CU.)
      f32x4 xs[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) xs[g] = mfma16(sx[g], neg136, zero4);
      f32x4 pr[2];
      float scv[2];
      auto product = [&](int i) {
        const int g = i / NTW, nt = i % NTW;
        const u32x4 wb = unpack_128q(s.w[nt][g]);
        const uint32_t sw = s.s[nt][g >> 1];
        scv[i & 1] = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
        pr[i & 1] = mfma16(sx[g], wb, xs[g]);
      };
      auto scale = [&](int i) {
        const int nt = i % NTW;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[nt][r] = __builtin_fmaf(scv[i & 1], pr[i & 1][r], acc[nt][r]);
      };
      product(0);
#pragma unroll
      for (int i = 1; i < 4 * NTW; ++i) {
        product(i);
        scale(i - 1);
      }
      scale(4 * NTW - 1);
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 xs = mfma16(sx[g], neg136, zero4);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const u32x4 wb = unpack_128q(s.w[nt][g]);
          const uint32_t sw = s.s[nt][g >> 1];
          const float scv = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
          const f32x4 pr = mfma16(sx[g], wb, xs);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nt][r] = __builtin_fmaf(scv, pr[r], acc[nt][r]);
        }
      }
    }
    if (++c_c == KC) {
      // column block c_nb complete: lane holds rows 4*kb + r of column col
      if (p.act) {
#pragma unroll
        for (int nt = 0; nt < NTW; nt += 2) {
          const int n = (((c_nb * 4 + w) * NTW + nt) / 2) * 16 + col;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (out_row[r] >= 0)
              p.c[(size_t)out_row[r] * (p.N / 2) + n] =
                  fused_silu_mul(acc[nt][r] * tw[r], acc[nt + 1][r] * tw[r]);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int n = ((c_nb * 4 + w) * NTW + nt) * 16 + col;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (out_row[r] >= 0)
              p.c[(size_t)out_row[r] * p.N + n] =
                  (uint16_t)(pack_bf16x2(acc[nt][r] * tw[r], 0.f) & 0xFFFFu);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] = 0.f;
      c_c = 0;
      ++c_nb;
    }
  };

  // Same pipeline as the kernel above, over the flattened stream.
  int f = 0;
  if (total >= 2 * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      __builtin_amdgcn_sched_barrier(0);
      load_next(st[d]);
    }
    for (; f + 2 * D <= total; f += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        __builtin_amdgcn_sched_barrier(0);
        step(st[d], d);
        __builtin_amdgcn_sched_barrier(0);
        load_next(st[d]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < total) load_next(st[d]);
  }
  for (; f < total; f += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (f + d < total) {
        step(st[d], d);
        if (f + d + D < total) load_next(st[d]);
      }
    }
  }
}

// Small-M variant with the token rows shared by the workgroup: TM 16-token
// tiles and one column block of 64 * NTW columns, the four waves side by
// side over 16 * NTW columns each. Without split-K a workgroup runs the
// whole K; with it, workgroup sp of a (tile, column block) runs the sp-th K
// range and writes fp32 partials for the ordered reduction. A chunk's token
// rows (TM * 16 rows x 256 bytes) go through a ring of D LDS buffers, each
// wave copying a quarter of them with direct-to-LDS loads (slot j of row r
// holds segment j ^ (r % 16)); weights go through D register stages per
// wave. One bare barrier per chunk: at step j every wave has its own loads
// of chunk j (wait count) and, past the barrier, every wave is done with
// chunk j-1, whose buffer then takes chunk j+D-1. Sharing the rows keeps the
// LDS (D * TM * 4 KiB) and register budget small enough for three
// workgroups per CU, which decode grids need to keep HBM busy, and loads
// each row once per workgroup instead of once per wave.
template <int TM, int D>
constexpr int xs_lds_bytes() { return D * TM * 16 * 256 + TM * 16 * 8; }

template <int NTW>
struct XsStage {
  u32x4 w[NTW];
  u32x2 s[NTW];
};

// One 128-wide K chunk of the shared-row kernels. The chunk's token rows
// sit in LDS at xb (row r of tile tm at xb + (tm * 16 + r) * 256, segment
// j of a row in slot j ^ (r % 16)), the wave's weight words and scales in
// st; the products accumulate into acc (lane l: rows 4 * (l / 16) + i of
// column l % 16 of each 16 x 16 tile).
template <int TM, int NTW>
__device__ __forceinline__ void xs_compute(f32x4 (&acc)[NTW][TM], const XsStage<NTW>& st,
                                           uint32_t xb, int kb, int col) {
  constexpr int XROW = 256;
  const u32x4 neg136 = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // Four token tiles share each weight word: dequantising it once to
  // bf16((q - 8) s) (about 19 VALU) then costs less than the exact form's
  // per-tile scale FMAs (4 per tile) and zero-point MFMAs, and the MFMAs
  // accumulate straight into acc. Fewer tiles keep the exact form.
  constexpr bool kScaledW = TM >= 4;
  if constexpr (TM == 1 && NTW == 4) {
    // One token tile, four column tiles: the chunk's four fragments are
    // read at once and their four zero-point MFMAs go first, so no
    // product waits on the one just before it; products and scale FMAs
    // then run pipelined by one over the chunk's (group, column tile)
    // pairs. Same operations per accumulator, in the same order, as the
    // general form below. (EP8 decode gate_up 132.6-133.1 -> 130.3-130.6
    // us; with two column tiles the TP8 gate_up share ran 2.6 % slower
    // than the general form, so that instance keeps it.)
    u32x4 xg[4];
    static_for<4>([&](auto g) { xg[g] = lds_read16<0>(xb + (((4 * g + kb) ^ col) << 4)); });
    static_for<4>([&](auto g) { wait_lgkm<3 - g>(xg[g]); });
    f32x4 xsum[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) xsum[g] = mfma16(xg[g], neg136, zero4);
    f32x4 pr[2];
    float scv[2];
    auto product = [&](int i) {
      const int g = i / NTW, nt = i % NTW;
      const u32x4 wb = unpack_128q(st.w[nt][g]);
      const uint32_t sw = st.s[nt][g >> 1];
      scv[i & 1] = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
      pr[i & 1] = mfma16(xg[g], wb, xsum[g]);
    };
    auto scale = [&](int i) {
      const int nt = i % NTW;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[nt][0][r] = __builtin_fmaf(scv[i & 1], pr[i & 1][r], acc[nt][0][r]);
    };
    product(0);
#pragma unroll
    for (int i = 1; i < 4 * NTW; ++i) {
      product(i);
      scale(i - 1);
    }
    scale(4 * NTW - 1);
    return;
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t a = xb + (((4 * g + kb) ^ col) << 4);
    u32x4 xg[TM];
    static_for<TM>([&](auto tm) { xg[tm] = lds_read16<tm * 16 * XROW>(a); });
    static_for<TM>([&](auto tm) { wait_lgkm<TM - 1 - tm>(xg[tm]); });
    if constexpr (kScaledW) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const uint32_t sw = st.s[nt][g >> 1];
        const float scv = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
        const u32x4 wb = dequant8(st.w[nt][g], scv, -8.0f * scv);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[nt][tm] = mfma16(xg[tm], wb, acc[nt][tm]);
      }
      continue;
    }
    f32x4 xsum[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) xsum[tm] = mfma16(xg[tm], neg136, zero4);
    // Pipelined by one column tile: tile nt's products are issued before
    // tile nt-1's scale FMAs, so the FMAs run while the matrix core works
    // instead of waiting out each product's latency. Every accumulator
    // takes the same operations in the same order as the plain loop
    // (kept for reference and for instances that would not fit).
    if constexpr (TM * NTW > 8) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const u32x4 wb = unpack_128q(st.w[nt][g]);
        const uint32_t sw = st.s[nt][g >> 1];
        const float sc = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const f32x4 p1 = mfma16(xg[tm], wb, xsum[tm]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nt][tm][r] = __builtin_fmaf(sc, p1[r], acc[nt][tm][r]);
        }
      }
      continue;
    }
    f32x4 pr[2][TM];
    float scv[2];
    auto product = [&](int nt) {
      const u32x4 wb = unpack_128q(st.w[nt][g]);
      const uint32_t sw = st.s[nt][g >> 1];
      scv[nt & 1] = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) pr[nt & 1][tm] = mfma16(xg[tm], wb, xsum[tm]);
    };
    auto scale = [&](int nt) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[nt][tm][r] = __builtin_fmaf(scv[nt & 1], pr[nt & 1][tm][r], acc[nt][tm][r]);
    };
    product(0);
#pragma unroll
    for (int nt = 1; nt < NTW; ++nt) {
      product(nt);
      scale(nt - 1);
    }
    scale(NTW - 1);
  }
}

// One (token tile, column block, K split) of the shared-row kernel; s_x
// holds xs_lds_bytes<TM, D>() bytes of LDS: the D token buffers, then the
// tile's output rows and topk weights (TM * 16 of each).
template <int TM, int NTW, int D>
__device__ __forceinline__ void xs_tile(const GemmParams& p, int tile, int nb, int sp,
                                        uint8_t* s_x, int tid) {
  constexpr int XROW = 256;
  constexpr int XBUF = TM * 16 * XROW;       // one chunk of the tile's token rows
  constexpr int NX = TM;                     // direct-to-LDS loads per wave and chunk
  constexpr int NW = 2 * NTW;                // weight + scale loads per wave and chunk
  static_assert(D >= 2, "pipeline depth");
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kb = lane >> 4;
  // Indexed routing: the slots of the rows this lane will look up are read
  // together with the tile's expert, so that the first token-row loads wait
  // one memory round trip rather than two.
  int sid_x[NX], sid_t = -1;
  if (p.mode == 0) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int pos = tile * p.BM + 4 * (w * NX + i) + kb;
      sid_x[i] = pos < p.cap ? p.sorted_ids[pos] : -1;
    }
    if (w == 0 && lane < TM * 16) {
      const int pos = tile * p.BM + lane;
      sid_t = pos < p.cap ? p.sorted_ids[pos] : -1;
    }
  }
  const int e = __builtin_amdgcn_readfirstlane(tile_expert(p, tile));
  if (e < 0) return;
  // row_info from a slot read above (indexed routing), else looked up
  auto row_of = [&](int sid, int row) __attribute__((always_inline)) {
    if (p.mode != 0) return row_info(p, tile, e, row);
    RowInfo ri{false, 0, 0};
    if (sid >= 0 && sid < p.num_slots) {
      ri.valid = true;
      ri.a_row = sid / p.a_row_div;
      ri.out_row = sid;
    }
    return ri;
  };
  const int KC = p.KC;
  // this workgroup's K range (all of K without split-K; the host keeps
  // split_k <= K / 128, so every range holds a chunk)
  const int cs0 = (int)(((int64_t)sp * KC) / p.split);
  const int total = (int)(((int64_t)(sp + 1) * KC) / p.split) - cs0;
  if (total <= 0) return;

  // weights and scales of this column block: wave w owns its 16-column
  // tiles (nb * 4 + w) * NTW + nt
  const int nt0 = nb * 4 * NTW;
  const uint32_t tile_bytes = (uint32_t)KC * kWBlockBytes;
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(p.wpk + (size_t)e * p.NT * tile_bytes, (uint32_t)p.NT * tile_bytes);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(p.spk + (size_t)e * p.NT * KC * kSBlockBytes, (uint32_t)p.NT * KC * kSBlockBytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
  const TileAddr wa = tile_addr(p, nt0 + w * NTW, kWBlockBytes);
  const TileAddr sa = tile_addr(p, nt0 + w * NTW, kSBlockBytes);
  const uint32_t voff_w = lane * 16 + wa.base;
  const uint32_t voff_s = col * 8 + sa.base;
  // wave w copies rows 4 (w * NX + i) + l / 16, i < NX
  uint32_t voff_x[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int row = 4 * (w * NX + i) + kb;
    const RowInfo ri = row_of(sid_x[i], row);
    const uint32_t seg = (uint32_t)(col ^ (row & 15));
    voff_x[i] = ri.valid ? (uint32_t)ri.a_row * (uint32_t)p.K * 2u + seg * 16u : 0x80000000u;
  }
  // The tile's output rows and topk weights: wave 0 looks them up here,
  // so that the loads overlap the pipeline's start, and parks them in LDS
  // after the prologue; the K loop holds no registers for them.
  int32_t* s_orow = (int32_t*)(s_x + D * XBUF);
  float* s_tw = (float*)(s_orow + TM * 16);
  const bool scale_rows = p.split == 1 && p.mode == 0 && p.topk_w;
  int32_t my_orow = -1;
  float my_tw = 1.0f;
  if (w == 0 && lane < TM * 16) {
    const RowInfo ri = row_of(sid_t, lane);
    my_orow = ri.valid ? ri.out_row : -1;
    my_tw = (ri.valid && scale_rows) ? p.topk_w[ri.out_row] : 1.0f;
  }

  // step f -> K chunk; past the end the last chunk is fetched again, so
  // every step issues the same loads
  auto chunk = [&](int f) { return cs0 + min(f, total - 1); };
  auto load_w = [&](XsStage<NTW>& st, int f) {
    const int c = chunk(f);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      st.w[nt] = __builtin_amdgcn_raw_buffer_load_b128(rw, voff_w, nt * wa.tile + c * wa.chunk,
                                                       kNonTemporal);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      st.s[nt] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff_s, nt * sa.tile + c * sa.chunk, 0);
  };
  auto load_x = [&](auto buf_id, int f) {
    constexpr int b = decltype(buf_id)::value;
    const int c = chunk(f);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int vo = (int)voff_x[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra,
          (__attribute__((address_space(3))) void*)(s_x + b * XBUF + 4 * (w * NX + i) * XROW),
          16, vo, c * XROW, 0, 0);
    }
  };

  f32x4 acc[NTW][TM];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) acc[nt][tm] = f32x4{0.f, 0.f, 0.f, 0.f};
  // operand read: row tm*16 + l%16, segment 4g + l/16 at slot segment ^ (l%16)
  const uint32_t xrd = lds_addr(s_x) + col * XROW;

  auto compute = [&](auto buf_id, const XsStage<NTW>& st) {
    constexpr int b = decltype(buf_id)::value;
    xs_compute<TM, NTW>(acc, st, xrd + b * XBUF, kb, col);
  };

  // Pipeline. Issue order: prologue W(0) X(0) W(1) X(1) .. X(D-2) W(D-1);
  // step j: [wait, barrier] X(j+D-1) into the buffer of chunk j-1, compute
  // chunk j, W(j+D). When step j waits, the loads issued after X(j) are
  // W(j+1) and D-2 pairs (X, W): that count is exact on every step.
  constexpr int kAfter = NW + (D - 2) * (NX + NW);
  XsStage<NTW> ws[D];
  static_for<D - 1>([&](auto d) {
    load_w(ws[d], d);
    load_x(d, d);
    __builtin_amdgcn_sched_barrier(0);
  });
  load_w(ws[D - 1], D - 1);
  if (w == 0 && lane < TM * 16) {
    s_orow[lane] = my_orow;
    s_tw[lane] = my_tw;
  }
  auto step = [&](int j, auto cur) {
    constexpr int b = decltype(cur)::value;
    wait_vmcnt<kAfter>();
    lds_barrier();
    load_x(std::integral_constant<int, (b + D - 1) % D>{}, j + D - 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, ws[b]);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ws[b], j + D);
  };
  // Whole rounds of D steps, then the last total % D. Every step of the
  // loop body runs unconditionally: a step that could be skipped inside the
  // loop would let the compiler assume a path on which the next step's
  // weights have fewer loads behind them, and it would then wait for the
  // stage issued one step ahead before computing.
  int j = 0;
  for (; j + D <= total; j += D) static_for<D>([&](auto d) { step(j + d, d); });
  static_for<D - 1>([&](auto d) {
    if (j + d < total) step(j + d, d);
  });
  wait_vmcnt<0>();
  // every wave's view of the row table (a one-chunk range has had no
  // barrier since wave 0 wrote it)
  __syncthreads();

  // Output: lane holds rows tm*16 + 4*kb + r of column col of each tile.
  if (p.act && p.split == 1) {
    // fused activation: tiles nt (gate) and nt + 1 (up) of each pair
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const i32x4 orow = *(const i32x4*)(s_orow + tm * 16 + kb * 4);
      const f32x4 twv = *(const f32x4*)(s_tw + tm * 16 + kb * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (orow[r] < 0) continue;
#pragma unroll
        for (int nt = 0; nt < NTW; nt += 2)
          p.c[(size_t)orow[r] * (p.N / 2) + ((nt0 + w * NTW + nt) / 2) * 16 + col] =
              fused_silu_mul(acc[nt][tm][r] * twv[r], acc[nt + 1][tm][r] * twv[r]);
      }
    }
    return;
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const i32x4 orow = *(const i32x4*)(s_orow + tm * 16 + kb * 4);
    const f32x4 twv = *(const f32x4*)(s_tw + tm * 16 + kb * 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (orow[r] < 0) continue;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int n = (nt0 + w * NTW + nt) * 16 + col;
        if (p.split > 1)
          p.ws[((size_t)sp * p.rows_cap + orow[r]) * p.N + n] = acc[nt][tm][r];
        else
          p.c[(size_t)orow[r] * p.N + n] =
              (uint16_t)(pack_bf16x2(acc[nt][tm][r] * twv[r], 0.f) & 0xFFFFu);
      }
    }
  }
}

// Semi-static schedule: the grid covers every (tile, column group) the
// host can bound; a workgroup derives its item from its index and the
// routing buffers, and items past the routed ones exit at once.
// Four workgroups per CU (at most 128 VGPRs), except the 32-row, 4-tile
// instance: its pipelined products need 140, and at three per CU it ran the
// masked gate_up share 3 % faster and its down share 1 % slower than the
// plain order at four.
template <int TM, int NTW>
constexpr int xs_occupancy() { return (TM == 2 && NTW == 4) ? 3 : 4; }

template <int TM, int NTW, int D>
__global__ __launch_bounds__(256, (xs_occupancy<TM, NTW>())) void gemm_small_m_xs_kernel(
    const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_x[xs_lds_bytes<TM, D>()];
  int tile, grp, sp;
  if (!decode_bid(p, blockIdx.x, tile, grp, sp)) return;
  xs_tile<TM, NTW, D>(p, tile, grp, sp, s_x, (int)threadIdx.x);
}

// Dynamic schedule: a persistent grid whose workgroups take (tile, column
// group) items from the work counter until the routed items run out.
template <int TM, int NTW, int D>
__global__ __launch_bounds__(256, 3) void gemm_small_m_xs_dyn_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_x[xs_lds_bytes<TM, D>()];
  __shared__ int s_item;
  const int ntiles = p.mode == 0 ? min(*p.ntp / p.BM, p.num_tiles) : p.num_tiles;
  const int items = ntiles * p.nblocks;
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(p.work, 1);
    __syncthreads();
    const int it = __builtin_amdgcn_readfirstlane(s_item);
    if (it >= items) break;
    const int tile = it / p.nblocks;
    xs_tile<TM, NTW, D>(p, tile, it - tile * p.nblocks, 0, s_x, (int)threadIdx.x);
    // every wave is done with s_item and the LDS ring before the next item
    __syncthreads();
  }
}

// Gang schedule: a persistent grid whose workgroups hold S groups of four
// waves, each group running its own (tile, column block, split) item. The
// groups share the per-chunk barrier, so the items of a workgroup advance in
// lock-step and end together. Separate workgroups on one CU do not: the
// oldest is issued first and finishes early, and the CU then streams with
// fewer loads in flight. Items keep the XCD-aware order: group g of
// workgroup b takes the items k = (b / 8) * S + g, then k + S * grid / 8,
// ... of XCD b % 8.
template <int TM, int D>
constexpr int xs_gang_stride() { return (xs_lds_bytes<TM, D>() + 1023) / 1024 * 1024; }

template <int TM, int NTW, int D, int S>
__global__ __launch_bounds__(256 * S, 1) void gemm_small_m_xs_gang_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_x[S * xs_gang_stride<TM, D>()];
  const int g = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 8));
  const int tid = (int)(threadIdx.x & 255);
  const int xcd = blockIdx.x & 7;
  const int step = (int)(gridDim.x >> 3) * S;
  for (int k = (int)(blockIdx.x >> 3) * S + g;; k += step) {
    int tile, nb, sp;
    if (!decode_bid(p, k * 8 + xcd, tile, nb, sp)) break;
    xs_tile<TM, NTW, D>(p, tile, nb, sp, s_x + g * xs_gang_stride<TM, D>(), tid);
    // the group's LDS ring and row table are free for its next item
    __syncthreads();
  }
}

// Stream-K gang schedule: one workgroup of S four-wave groups per CU, each
// CU taking a contiguous share of the (token tile, column block) items,
// balanced to one item over the CUs. Inside the workgroup the share's K
// chunks are split evenly over the groups, so an item can be cut in K
// between neighbouring groups; the groups advance in lock-step through
// the per-chunk barrier and end together, and no CU idles at the end of
// the launch as a semi-static grid's last round leaves it. A group walks
// its chunks as one stream through the shared-row pipeline: the next
// item's loads are in flight while the current one finishes. A finished
// item stays in the accumulators and is stored at the next step, ahead of
// that step's loads, so the pipeline's wait counts never include stores.
// An item cut in K: the group holding its first chunk (the owner) keeps
// its piece in registers to the end; a group whose range starts inside
// the item leaves its piece as fp32 in its LDS slot, and after the final
// barrier the owner adds the later pieces in K order (the ordered split
// reduction of split-K, inside one workgroup). Items are ordered token
// tile by column block, and the CU shares of one XCD are contiguous, so a
// tile's token rows stay in few L2s. Indexed (moe_align) routing only;
// the host keeps every group's range within two token tiles.
template <int TM, int NTW>
constexpr int sk_group_bytes() {
  return (2 * TM * 16 * 256 + 2 * TM * 16 * 8 + TM * 16 * 64 * NTW * 4 + 1023) / 1024 * 1024;
}

__device__ __forceinline__ void lds_write16(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// The body of the stream-K kernel; lds holds S * sk_group_bytes<TM, NTW>()
// bytes: per group its token ring, the row tables of two tiles and its slot.
template <int TM, int NTW, int S>
__device__ __forceinline__ void sk_workgroup(const GemmParams& p, uint8_t* lds) {
  constexpr int D = 2;
  constexpr int XROW = 256;
  constexpr int XBUF = TM * 16 * XROW;
  constexpr int NX = TM;
  constexpr int NW = 2 * NTW;
  constexpr int ROWS = TM * 16;
  constexpr int GB = sk_group_bytes<TM, NTW>();
  static_assert(2 * ROWS <= 64 && NTW % 2 == 0, "row tables of two tiles come from one wave");
  const int g = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 8));
  const int tid = (int)(threadIdx.x & 255);
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kb = lane >> 4;
  uint8_t* s_x = lds + g * GB;
  int32_t* s_orow = (int32_t*)(s_x + D * XBUF);  // [2][ROWS]: output rows of the two tiles
  float* s_tw = (float*)(s_orow + 2 * ROWS);     // [2][ROWS]: their topk weights
  // fp32 piece of group k in lane layout: f32x4 (w, tm, nt) at lane * 16
  auto slot_addr = [&](int k, int tm, int nt) __attribute__((always_inline)) {
    return lds_addr(lds) + (uint32_t)(k * GB + D * XBUF + 2 * ROWS * 8 +
                                      ((w * TM + tm) * NTW + nt) * 1024 + lane * 16);
  };

  // This workgroup's items [i0, i1) and this group's units (K chunks,
  // counted from item i0's first chunk) [ua, ub).
  const int KC = p.KC, nbl = p.nblocks;
  const int ntiles = min(*p.ntp / p.BM, p.num_tiles);
  const int64_t items = (int64_t)max(ntiles, 0) * nbl;
  const int grid = (int)gridDim.x;
  const int rk = (int)(blockIdx.x & 7) * (grid >> 3) + (int)(blockIdx.x >> 3);
  const int64_t i0 = items * rk / grid, i1 = items * (rk + 1) / grid;
  if (i0 >= i1) return;
  const int64_t U = (i1 - i0) * KC;
  auto ustart = [&](int k) __attribute__((always_inline)) { return (int)(U * k / S); };
  const int ua = ustart(g), ub = ustart(g + 1);
  const int n = ub - ua;                    // >= 2: U >= KC >= 8 > S
  const int nmax = (int)((U + S - 1) / S);  // steps of the longest group
  const int64_t ia = i0 + ua / KC, ib = i0 + (ub - 1) / KC;
  const int tA = (int)(ia / nbl), tB = (int)(ib / nbl);
  const int eA = __builtin_amdgcn_readfirstlane(tile_expert(p, tA));
  const int eB = __builtin_amdgcn_readfirstlane(tile_expert(p, tB));

  // weights and scales of the two tiles' experts (none for a tile whose
  // expert id is out of range: its items then read zeros and store nothing)
  const uint32_t wbytes = (uint32_t)p.NT * KC * kWBlockBytes;
  const uint32_t sbytes = (uint32_t)p.NT * KC * kSBlockBytes;
  const __amdgpu_buffer_rsrc_t rwA = make_rsrc(p.wpk + (size_t)max(eA, 0) * wbytes, eA >= 0 ? wbytes : 0u);
  const __amdgpu_buffer_rsrc_t rwB = make_rsrc(p.wpk + (size_t)max(eB, 0) * wbytes, eB >= 0 ? wbytes : 0u);
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.spk + (size_t)max(eA, 0) * sbytes, eA >= 0 ? sbytes : 0u);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(p.spk + (size_t)max(eB, 0) * sbytes, eB >= 0 ? sbytes : 0u);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
  const uint32_t voff_w = lane * 16, voff_s = col * 8;
  // token rows: wave w copies rows 4 (w * NX + i) + l / 16 of the tile
  uint32_t vxA[NX], vxB[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int row = 4 * (w * NX + i) + kb;
    const uint32_t seg = (uint32_t)(col ^ (row & 15));
    const RowInfo r0 = row_info(p, tA, eA, row), r1 = row_info(p, tB, eB, row);
    vxA[i] = (r0.valid && eA >= 0) ? (uint32_t)r0.a_row * (uint32_t)p.K * 2u + seg * 16u
                                   : 0x80000000u;
    vxB[i] = (r1.valid && eB >= 0) ? (uint32_t)r1.a_row * (uint32_t)p.K * 2u + seg * 16u
                                   : 0x80000000u;
  }
  // output rows and topk weights of both tiles: wave 0 looks them up here
  // and parks them in LDS after the prologue
  int32_t my_orow = -1;
  float my_tw = 1.0f;
  if (w == 0 && lane < 2 * ROWS) {
    const bool second = lane >= ROWS;
    const int t = second ? tB : tA, e = second ? eB : eA;
    const RowInfo ri = row_info(p, t, e, lane - (second ? ROWS : 0));
    my_orow = (ri.valid && e >= 0) ? ri.out_row : -1;
    my_tw = (ri.valid && e >= 0 && p.mode == 0 && p.topk_w) ? p.topk_w[ri.out_row] : 1.0f;
  }

  // Cursor over the group's units: K chunk, column block and token tile
  // (0: tA, 1: tB) of the next unit to load or compute. It stays on the
  // last unit once there, so loads past the end fetch that unit again.
  struct Cursor {
    int c, nb, t, left;
  };
  auto advance = [&](Cursor& q) __attribute__((always_inline)) {
    if (q.left > 1) {
      --q.left;
      if (++q.c == KC) {
        q.c = 0;
        if (++q.nb == nbl) {
          q.nb = 0;
          q.t = 1;
        }
      }
    }
  };
  const Cursor c0{ua % KC, (int)(ia % nbl), 0, n};
  Cursor wcur = c0, xcur = c0, ccur = c0;

  auto load_w = [&](XsStage<NTW>& st) __attribute__((always_inline)) {
    const int t0 = (wcur.nb * 4 + w) * NTW;
    const TileAddr wa = tile_addr(p, t0, kWBlockBytes), sa = tile_addr(p, t0, kSBlockBytes);
    const __amdgpu_buffer_rsrc_t rw = wcur.t ? rwB : rwA;
    const __amdgpu_buffer_rsrc_t rs = wcur.t ? rsB : rsA;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      st.w[nt] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, voff_w, wa.base + nt * wa.tile + wcur.c * wa.chunk, kNonTemporal);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      st.s[nt] = __builtin_amdgcn_raw_buffer_load_b64(
          rs, voff_s, sa.base + nt * sa.tile + wcur.c * sa.chunk, 0);
    advance(wcur);
  };
  auto load_x = [&](auto buf_id) __attribute__((always_inline)) {
    constexpr int b = decltype(buf_id)::value;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const uint32_t vo = xcur.t ? vxB[i] : vxA[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra,
          (__attribute__((address_space(3))) void*)(s_x + b * XBUF + 4 * (w * NX + i) * XROW),
          16, (int)vo, xcur.c * XROW, 0, 0);
    }
    advance(xcur);
  };

  f32x4 acc[NTW][TM];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc[nt][tm] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();
  const uint32_t xrd = lds_addr(s_x) + col * XROW;
  const uint32_t tbl = lds_addr(s_orow) + kb * 16;

  // Store the finished item in acc: rows 4 kb + r of column col of each
  // tile, scaled by the rows' topk weights and rounded to bf16 (with the
  // activation fused: output tile q from gate tile 2 q and up tile 2 q + 1).
  auto store_item = [&](int t, int nb) __attribute__((always_inline)) {
    const int t0 = (nb * 4 + w) * NTW;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      // LDS reads the compiler does not track (it would wait for every
      // direct-to-LDS load in flight before its own)
      u32x4 rv = lds_read16<0>(tbl + (uint32_t)((t * ROWS + tm * 16) * 4));
      u32x4 tv = lds_read16<0>(tbl + (uint32_t)((2 * ROWS + t * ROWS + tm * 16) * 4));
      wait_lgkm<0>(rv);
      wait_lgkm<0>(tv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int orow = (int)rv[r];
        const float twr = __uint_as_float(tv[r]);
        if (orow < 0) continue;
        if (p.act) {
#pragma unroll
          for (int q = 0; q < NTW / 2; ++q)
            p.c[(size_t)orow * (p.N / 2) + (t0 / 2 + q) * 16 + col] =
                fused_silu_mul(acc[2 * q][tm][r] * twr, acc[2 * q + 1][tm][r] * twr);
        } else {
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
            p.c[(size_t)orow * p.N + (t0 + nt) * 16 + col] =
                (uint16_t)(pack_bf16x2(acc[nt][tm][r] * twr, 0.f) & 0xFFFFu);
        }
      }
    }
  };
  auto put_slot = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        lds_write16(slot_addr(g, tm, nt), __builtin_bit_cast(u32x4, acc[nt][tm]));
  };

  // Pipeline (as the shared-row kernel, D = 2): prologue W(0) X(0) W(1);
  // step j: [wait, barrier] the store of an item finished at step j - 1
  // (still in acc), X(j+1) into the buffer of chunk j - 1, chunk j,
  // W(j+2). When step j waits, only W(j+1) was issued after X(j): stores
  // go out ahead of the step's loads, so the count holds.
  XsStage<NTW> ws[D];
  load_w(ws[0]);
  load_x(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  load_w(ws[1]);
  if (w == 0 && lane < 2 * ROWS) {
    s_orow[lane] = my_orow;
    s_tw[lane] = my_tw;
    // written before the first (bare) barrier lets other waves read them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  bool from0 = c0.c == 0;  // the piece in acc began at its item's first chunk
  bool pend = false;
  int pend_t = 0, pend_nb = 0;
  auto step = [&](int j, auto cur) __attribute__((always_inline)) {
    constexpr int b = decltype(cur)::value;
    wait_vmcnt<NW>();
    lds_barrier();
    if (pend) {
      store_item(pend_t, pend_nb);
      zero_acc();
      pend = false;
    }
    __builtin_amdgcn_sched_barrier(0);
    load_x(std::integral_constant<int, b ^ 1>{});
    __builtin_amdgcn_sched_barrier(0);
    if (j < n) {
      xs_compute<TM, NTW>(acc, ws[b], xrd + b * XBUF, kb, col);
      if (j < n - 1 && ccur.c == KC - 1) {
        // an item's last chunk: a whole item stays in acc for the store at
        // the next step; a piece that began inside the item goes to the
        // slot for its owner
        if (from0) {
          pend = true;
          pend_t = ccur.t;
          pend_nb = ccur.nb;
        } else {
          put_slot();
          zero_acc();
        }
        from0 = true;
      }
      advance(ccur);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_w(ws[b]);
  };
  // both steps of the loop body unconditional (see the shared-row kernel)
  int j = 0;
  for (; j + 2 <= nmax; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    step(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < nmax) step(j, std::integral_constant<int, 0>{});
  wait_vmcnt<0>();
  // The last piece: a whole item is stored; a piece that began inside its
  // item goes to the slot; the owner of an item that continues in the next
  // groups adds their pieces (each began inside the item) in K order.
  if (!from0) put_slot();
  // the slot writes are inline asm, which the barrier's own wait may not
  // count
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
  if (!from0) return;
  if (ccur.c != KC - 1) {
    const int xe = ((ub - 1) / KC + 1) * KC;  // end of the item, in units
    for (int k = g + 1; k < S; ++k) {
      if (ustart(k) >= xe) break;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          u32x4 v = lds_read16<0>(slot_addr(k, tm, nt));
          wait_lgkm<0>(v);
          acc[nt][tm] += __builtin_bit_cast(f32x4, v);
        }
      if (ustart(k + 1) >= xe) break;
    }
  }
  store_item(ccur.t, ccur.nb);
}

template <int TM, int NTW, int S>
__global__ __launch_bounds__(256 * S, 1) void gemm_small_m_sk_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * sk_group_bytes<TM, NTW>()];
  sk_workgroup<TM, NTW, S>(p, lds);
}

__global__ void reset_counter_kernel(int32_t* c) {
  if (threadIdx.x == 0) *c = 0;
}

// Static device scratch for callers that cannot allocate: every device the
// library runs on holds its own copy until the process ends. In host code the
// name below is only a stand-in for the symbol, never a device address; the
// address is looked up per device with hipGetSymbolAddress and only that
// pointer is handed to kernels.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;

int scratch_device_ptr(void** out) {
  static std::atomic<void*> ptrs[kMaxScratchDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxScratchDevices) return (int)hipErrorInvalidDevice;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = ptrs[dev].load(std::memory_order_relaxed);
    if (!p) {
      // the device is current here, so this is its copy of the array
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return (int)e;
      if (!p) return (int)hipErrorInvalidSymbol;
      ptrs[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return 0;
}

// Split-K reduction: c[row] = bf16( sum_s ws[s][row] (* topk weight) ), the
// splits summed in order ([release] indexed techniques: the split/reduce
// that the stream-K gate avoids on saturated grids). One thread per
// (row position, 4 columns).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmParams p) {
  if (p.act) {
    // fused activation: four outputs h[row, o0 .. o0+3] per thread, from
    // gate columns 32 q + c .. and up columns 32 q + 16 + c .. of the
    // partials (q = o0 / 16, c = o0 % 16)
    const int64_t per_row = p.N / 8;
    const int64_t total = (int64_t)p.num_tiles * p.BM * per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
      const int pos = (int)(i / per_row);
      const int o0 = (int)(i - (int64_t)pos * per_row) * 4;
      const int tile = pos / p.BM;
      const int e = tile_expert(p, tile);
      if (e < 0) continue;
      const RowInfo ri = row_info(p, tile, e, pos - tile * p.BM);
      if (!ri.valid) continue;
      const int ng = (o0 >> 4) * 32 + (o0 & 15);
      float4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < p.split; ++k) {
        const float* row = p.ws + ((size_t)k * p.rows_cap + ri.out_row) * p.N;
        const float4 a = *(const float4*)(row + ng);
        const float4 b = *(const float4*)(row + ng + 16);
        g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
        u.x += b.x; u.y += b.y; u.z += b.z; u.w += b.w;
      }
      const float t = (p.mode == 0 && p.topk_w) ? p.topk_w[ri.out_row] : 1.0f;
      u32x2 o;
      o.x = (uint32_t)fused_silu_mul(g.x * t, u.x * t) |
            ((uint32_t)fused_silu_mul(g.y * t, u.y * t) << 16);
      o.y = (uint32_t)fused_silu_mul(g.z * t, u.z * t) |
            ((uint32_t)fused_silu_mul(g.w * t, u.w * t) << 16);
      *(u32x2*)(p.c + (size_t)ri.out_row * (p.N / 2) + o0) = o;
    }
    return;
  }
  const int64_t per_row = p.N / 4;
  const int64_t total = (int64_t)p.num_tiles * p.BM * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int pos = (int)(i / per_row);
    const int n0 = (int)(i - (int64_t)pos * per_row) * 4;
    const int tile = pos / p.BM;
    const int e = tile_expert(p, tile);
    if (e < 0) continue;
    const RowInfo ri = row_info(p, tile, e, pos - tile * p.BM);
    if (!ri.valid) continue;
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < p.split; ++k) {
      const float4 v = *(const float4*)(p.ws + ((size_t)k * p.rows_cap + ri.out_row) * p.N + n0);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    const float t = (p.mode == 0 && p.topk_w) ? p.topk_w[ri.out_row] : 1.0f;
    u32x2 o;
    o.x = pack_bf16x2(s.x * t, s.y * t);
    o.y = pack_bf16x2(s.z * t, s.w * t);
    *(u32x2*)(p.c + (size_t)ri.out_row * p.N + n0) = o;
  }
}

// ---------------------------------------------------------------------------
// Large-M expert GEMM (prefill shapes: 128-token tiles).
//
// Workgroup: 4 waves over one 128-token tile and 256 weight columns, each
// wave owning 64 columns for all 128 tokens as 4 x 2 tiles of 32 x 32
// (v_mfma_f32_32x32x16_bf16). The 32 x 32 form is chosen over 16 x 16 x 32
// because it leaves more issue slots per flop for the dequantisation VALU
// work and halves the token-fragment reads per weight column pair; this
// kernel is issue-bound on those, not on the matrix core.
//
// Token tile: passes through LDS in 128-wide K chunks, fetched by
// direct-to-LDS buffer loads (16 bytes per lane, four rows per instruction)
// into one of two buffers one chunk ahead, with one barrier per chunk. Slot
// j of LDS row r holds the row's 16-byte segment j ^ (r % 16), so the rows an
// operand read touches fall in distinct banks. Rows the tile does not use get
// an out-of-range offset and arrive as zeros without being read.
//
// Weights never pass through LDS. The packed layout is the 16-column one the
// small-M kernel reads (lane l of a 16x128 tile holds column l % 16, K rows
// 8(l/16)..+7 of each 32-row group); a 32 x 32 x 16 operand needs column
// l % 32, K rows 8(l/32)..+7 of a 16-row half, which is lane
// (l % 16) + 16 (2h + l/32) of 16-column tile (l % 32)/16, so each lane
// loads that lane's 16 bytes (one word per group) for h = 0 and 1. Words are
// dequantised in registers to bf16((q - 8) s): two nibbles at a time become
// exact floats (a byte holding q in 0..15, read as an OCP e4m3 code with
// power-of-two scale 512, is exactly q), then q s - 8 s is one fp32 FMA
// rounded once more to bf16. The cost is paid once per 128 tokens.
// ---------------------------------------------------------------------------
constexpr int kLmBM = 128;          // tokens per tile
constexpr int kLmBN = 256;          // columns per workgroup
constexpr int kLmRowBytes = 256;    // one 128-wide K chunk of a bf16 row
constexpr int kLmMT = kLmBM / 32;   // 32-row tiles per wave
constexpr int kLmNT = 2;            // 32-column tiles per wave
constexpr int kLmBLoads = 3 * kLmNT;  // weight + scale loads per chunk and wave

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Rows of a tile that hold no token are never computed: the tile's valid
// rows are counted first, and only the 32-row groups that hold any of them
// are loaded, multiplied and stored (a 128-row tile that ends an expert's
// rows typically holds fewer than 128). Each count of groups has its own
// copy of the main loop.
__global__ __launch_bounds__(256, 2) void gemm_large_m_kernel(const GemmParams p) {
  constexpr int BM = kLmBM;
  // Token-tile LDS buffers: two separate objects, so the compiler's wait
  // counts can tell a load into one buffer from a read of the other.
  __shared__ __attribute__((aligned(1024))) uint8_t s_a0[BM * kLmRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a1[BM * kLmRowBytes];
  __shared__ int32_t s_arow[BM];
  __shared__ int32_t s_out[BM];
  __shared__ int32_t s_rows;   // one past the tile's last valid row

  int tile, nb, sp;
  if (!decode_bid_lm(p, tile, nb, sp)) return;
  const int e = __builtin_amdgcn_readfirstlane(tile_expert(p, tile));
  if (e < 0) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c16 = lane & 15, kq = lane >> 5, l32 = lane & 31;

  if (threadIdx.x == 0) s_rows = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < BM; r += 256) {
    const RowInfo ri = row_info(p, tile, e, r);
    s_arow[r] = ri.valid ? ri.a_row : -1;
    s_out[r] = ri.valid ? ri.out_row : -1;
    if (ri.valid) atomicMax(&s_rows, r + 1);
  }
  __syncthreads();
  const int groups = __builtin_amdgcn_readfirstlane((s_rows + 31) >> 5);

  const int c0 = (int)(((int64_t)sp * p.KC) / p.split);
  const int c1 = (int)(((int64_t)(sp + 1) * p.KC) / p.split);
  const int n = c1 - c0;
  // chunk to fetch for step j; past the end the last chunk is fetched again
  // so every step issues the same loads and the wait counts stay exact
  auto chunk = [&](int j) { return c0 + min(j, n - 1); };

  // Weights: this wave's 64 columns are 16-column packed tiles nt16..+3;
  // 32-column tile t uses packed tiles 2t and 2t+1.
  const int nt16 = nb * (kLmBN / 16) + w * 4;
  const uint32_t tile_bytes = (uint32_t)p.KC * kWBlockBytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(
      uniform_ptr(p.wpk + (size_t)e * p.NT * tile_bytes), (uint32_t)p.NT * tile_bytes);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(uniform_ptr(p.spk + (size_t)e * p.NT * p.KC * kSBlockBytes),
                (uint32_t)p.NT * p.KC * kSBlockBytes);
  const TileAddr wa = tile_addr(p, nt16, kWBlockBytes), sa = tile_addr(p, nt16, kSBlockBytes);
  const int half16 = (lane >> 4) & 1;  // which 16-column tile of the 32
  const uint32_t voff_w = wa.base + half16 * wa.tile + (uint32_t)(c16 + 16 * kq) * 16u;
  const uint32_t voff_s = sa.base + half16 * sa.tile + c16 * 8;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(uniform_ptr(p.a), p.a_bytes);

  // The main loop and epilogue for a tile whose valid rows lie in its first
  // MT groups of 32.
  auto body = [&](auto mt_c) {
    constexpr int MT = decltype(mt_c)::value;  // 32-row groups computed
    constexpr int BMA = 32 * MT;               // rows loaded and computed
    constexpr int ROWS_W = BMA / 4;            // token rows each wave copies per chunk
    constexpr int NA = ROWS_W / 4;             // direct-to-LDS loads per lane per chunk
    // VALU work per K step is about 45 instructions whatever MT is; the
    // scheduling pattern spreads it over the step's 2 MT MFMAs.
    constexpr int VPM = MT == 4 ? 5 : (46 + 2 * MT - 1) / (2 * MT);

    // Token rows: wave w copies rows w*ROWS_W .. +ROWS_W-1, four rows (one
    // per 16-lane group) per instruction; lane l lands in slot l % 16 of its
    // row, which holds the row's segment (l % 16) ^ (row % 16).
    uint32_t voff_a[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = w * ROWS_W + 4 * i + (lane >> 4);
      const int ar = s_arow[row];
      const uint32_t seg = (uint32_t)(c16 ^ (row & 15));
      voff_a[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)p.K * 2u + seg * 16u : 0x80000000u;
    }
    // (the LDS address is formed from the __shared__ array itself, which the
    // host compilation pass can type-check)
    auto load_a = [&](auto buf_id, int c) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int off = (w * ROWS_W + 4 * i) * kLmRowBytes;
        const int vo = (int)voff_a[i];
        if constexpr (decltype(buf_id)::value == 0)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              ra, (__attribute__((address_space(3))) void*)(s_a0 + off), 16, vo,
              c * kLmRowBytes, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              ra, (__attribute__((address_space(3))) void*)(s_a1 + off), 16, vo,
              c * kLmRowBytes, 0, 0);
      }
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;

    struct BStage {
      u32x4 w[kLmNT][2];  // [32-column tile][K half]: one word per 32-row group
      u32x2 s[kLmNT];     // four group scales of the lane's column
    };
    auto load_b = [&](BStage& b, int c) {
#pragma unroll
      for (int t = 0; t < kLmNT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          b.w[t][h] = __builtin_amdgcn_raw_buffer_load_b128(
              rw, voff_w, 2 * t * wa.tile + c * wa.chunk + h * 512, 0);
#pragma unroll
      for (int t = 0; t < kLmNT; ++t)
        b.s[t] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff_s, 2 * t * sa.tile + c * sa.chunk, 0);
    };

    f32x16 acc[MT][kLmNT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < kLmNT; ++t) acc[mt][t] = f32x16{};

    // One chunk: 8 K steps of 16; step ks uses group g = ks / 2, half ks % 2.
    // Software-pipelined one step deep: the token fragments and dequantised
    // weights of step ks+1 are fetched and computed while step ks's MFMAs
    // run, so a wave alone on its SIMD does not wait out LDS latency.
    auto compute = [&](const uint8_t* abuf, const BStage& b) {
      auto frags = [&](u32x4 (&av)[MT], int ks) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int row = mt * 32 + l32;
          const int slot = (2 * ks + kq) ^ (row & 15);
          av[mt] = *(const u32x4*)(abuf + row * kLmRowBytes + slot * 16);
        }
      };
      auto deq = [&](u32x4 (&bw)[kLmNT], int ks) {
        const int g = ks >> 1, h = ks & 1;
#pragma unroll
        for (int t = 0; t < kLmNT; ++t) {
          const uint32_t sw = b.s[t][g >> 1];
          const float sc = (g & 1) ? bf16_hi(sw) : bf16_lo(sw);
          bw[t] = dequant8(b.w[t][h][g], sc, -8.0f * sc);
        }
      };
      u32x4 av[2][MT], bw[2][kLmNT];
      frags(av[0], 0);
      deq(bw[0], 0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int cur = ks & 1;
        if (ks < 7) {
          frags(av[cur ^ 1], ks + 1);
          deq(bw[cur ^ 1], ks + 1);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < kLmNT; ++t)
            acc[mt][t] = mfma32(av[cur][mt], bw[cur][t], acc[mt][t]);
        if (ks < 7) {
          // next step's fragment reads first, then each MFMA followed by a
          // share of the next step's dequantisation
          __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
#pragma unroll
          for (int i = 0; i < MT * kLmNT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          }
        }
      }
    };

    // Issue order per step j: [wait, barrier] token rows of chunk j+1 (into
    // the buffer chunk j-1 used), compute chunk j, weights of chunk j+2.
    // Chunk j's token rows are therefore followed by exactly chunk j+1's
    // weights (kLmBLoads loads) when step j waits for them.
    // A split that owns no K chunk (never planned; rejected on the host)
    // keeps its zero accumulators and stores zero partial sums.
    if (n > 0) {
    BStage bs0, bs1;
    load_b(bs0, chunk(0));
    load_a(B0{}, chunk(0));
    __builtin_amdgcn_sched_barrier(0);
    load_b(bs1, chunk(1));
    // step on chunk j: `cur` is j's buffer (0 or 1), the other gets chunk
    // j+1. The last step waits for everything, since the count of loads
    // issued after its token rows is not fixed there.
    auto step = [&](int j, auto cur, BStage& b) {
      if (j + 1 < n)
        wait_vmcnt<kLmBLoads>();
      else
        wait_vmcnt<0>();
      lds_barrier();
      // (sched barriers keep the weight prefetch behind the token-row loads)
      if constexpr (decltype(cur)::value == 0) {
        load_a(B1{}, chunk(j + 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(&s_a0[0], b);
      } else {
        load_a(B0{}, chunk(j + 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(&s_a1[0], b);
      }
      load_b(b, chunk(j + 2));
    };
    for (int j = 0;; j += 2) {
      step(j, B0{}, bs0);
      if (j + 1 >= n) break;
      step(j + 1, B1{}, bs1);
      if (j + 2 >= n) break;
    }
    wait_vmcnt<0>();
    }

    // Output. Accumulator element 4i + r of tile (mt, t) is token
    // 32 mt + 8 i + 4 (l/32) + r, column 32 t + l % 32 of the wave's 64;
    // direct stores would be 2-byte scatters. The tile goes through the two
    // token buffers instead (free once every wave is past its last read),
    // then out in full rows with 16-byte stores. Staged row R keeps its
    // 16-byte unit u at u ^ (R % 16), so the accumulator-layout writes (rows
    // 4 apart) and the row-major reads both fall in distinct banks.
    __syncthreads();
    if (p.split == 1) {
      // bf16 tile: BMA rows of 256 columns (512 bytes), rows 0..63 in s_a0
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int R = mt * 32 + 8 * i + 4 * kq + r;
            const int out = s_out[R];
            const float tw = (p.mode == 0 && p.topk_w && out >= 0) ? p.topk_w[out] : 1.0f;
            uint8_t* row = mt < kLmMT / 2 ? &s_a0[R * 512] : &s_a1[(R - BM / 2) * 512];
#pragma unroll
            for (int t = 0; t < kLmNT; ++t) {
              const int C = w * 64 + t * 32 + l32;
              *(uint16_t*)(row + (((C >> 3) ^ (R & 15)) << 4) + (C & 7) * 2) =
                  (uint16_t)(cvt_pk_bf16(acc[mt][t][4 * i + r] * tw, 0.f) & 0xFFFFu);
            }
          }
      __syncthreads();
      if (p.act) {
        // fused activation: 128 outputs per row, 8 per thread; output unit
        // v takes 16-byte units 4 (v/2) + v%2 (gate) and that + 2 (up) of
        // the staged row
        const int v = threadIdx.x & 15;
        const int ug = 4 * (v >> 1) + (v & 1);
#pragma unroll 4
        for (int it = 0; it < BMA / 16; ++it) {
          const int R = it * 16 + (threadIdx.x >> 4);
          const int out = s_out[R];
          const uint8_t* row = R < BM / 2 ? &s_a0[R * 512] : &s_a1[(R - BM / 2) * 512];
          const u32x4 gv = *(const u32x4*)(row + ((ug ^ (R & 15)) << 4));
          const u32x4 uv = *(const u32x4*)(row + (((ug + 2) ^ (R & 15)) << 4));
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = (uint32_t)(pack_bf16x2(silu_mul(bf16_lo(gv[q]), bf16_lo(uv[q])),
                                          silu_mul(bf16_hi(gv[q]), bf16_hi(uv[q]))));
          if (out >= 0) *(u32x4*)(p.c + (size_t)out * (p.N / 2) + nb * (kLmBN / 2) + v * 8) = o;
        }
      } else {
        const int u = threadIdx.x & 31;
#pragma unroll 4
        for (int it = 0; it < BMA / 8; ++it) {
          const int R = it * 8 + (threadIdx.x >> 5);
          const int out = s_out[R];
          const uint8_t* row = R < BM / 2 ? &s_a0[R * 512] : &s_a1[(R - BM / 2) * 512];
          const u32x4 v = *(const u32x4*)(row + ((u ^ (R & 15)) << 4));
          if (out >= 0) *(u32x4*)(p.c + (size_t)out * p.N + nb * kLmBN + u * 8) = v;
        }
      }
    } else {
      // fp32 partial sums: passes of up to BM/2 rows of 256 columns (1 KiB)
#pragma unroll
      for (int hp = 0; hp < (BMA + BM / 2 - 1) / (BM / 2); ++hp) {
        if (hp) __syncthreads();
#pragma unroll
        for (int mt = hp * kLmMT / 2; mt < min((hp + 1) * kLmMT / 2, MT); ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int L = mt * 32 + 8 * i + 4 * kq + r - hp * BM / 2;
              uint8_t* row = L < BM / 4 ? &s_a0[L * 1024] : &s_a1[(L - BM / 4) * 1024];
#pragma unroll
              for (int t = 0; t < kLmNT; ++t) {
                const int C = w * 64 + t * 32 + l32;
                *(float*)(row + (((C >> 2) ^ (L & 15)) << 4) + (C & 3) * 4) =
                    acc[mt][t][4 * i + r];
              }
            }
        __syncthreads();
        const int u = threadIdx.x & 63;
        constexpr int kPassRows = BM / 2;
#pragma unroll 4
        for (int it = 0; it < min(kPassRows, BMA - hp * kPassRows) / 4; ++it) {
          const int L = it * 4 + (threadIdx.x >> 6);
          const int out = s_out[hp * kPassRows + L];
          const uint8_t* row = L < BM / 4 ? &s_a0[L * 1024] : &s_a1[(L - BM / 4) * 1024];
          const u32x4 v = *(const u32x4*)(row + ((u ^ (L & 15)) << 4));
          if (out >= 0)
            *(u32x4*)(p.ws + ((size_t)sp * p.rows_cap + out) * p.N + nb * kLmBN + u * 4) = v;
        }
      }
    }
  };
  switch (groups) {
    case 0: break;   // no valid row: nothing to compute or store
    case 1: body(std::integral_constant<int, 1>{}); break;
    case 2: body(std::integral_constant<int, 2>{}); break;
    case 3: body(std::integral_constant<int, 3>{}); break;
    default: body(std::integral_constant<int, 4>{}); break;
  }
}

// ---------------------------------------------------------------------------
// Large-M expert GEMM, producer/consumer form (prefill and contiguous shapes;
// [release] performance highlights: the grouped kernels run a persistent main
// loop in which some warps load and dequantise while others run the matrix
// operations).
//
// One workgroup per CU with 16 waves: 8 consumers and 8 producers (two of
// each per SIMD). The grid is persistent. Workgroup (x = id % 8,
// slot = id / 8) walks the items (128-row tile, 256-column block) of the
// tiles dealt to XCD x (tiles x, x + 8, ...), taking every (G/8)-th item, so
// a tile's column blocks run on one XCD and share its token rows in that
// L2. The items of a workgroup form one stream of 64-wide K stages.
//
// Producers. Producer w owns 32-column tile w of the block and one 16-wide K
// step (w % 2) of 32 token rows (w / 2). Stages are 32 wide in K. Per stage
// a producer copies its token rows of the stage four ahead into LDS with a
// direct-to-LDS load (rows with no token arrive as zeros without being
// read), keeps its packed weights in registers up to eight stages ahead
// (three 128-wide chunks in flight), and dequantises the current stage's
// quarter chunk into LDS once for the whole workgroup, as bf16((q - 8) s)
// (the same rounding as the kernel above) laid
// out as 32 x 32 x 16 MFMA B fragments: for 32-column tile ct and K step ks,
// lane l's 16 bytes hold column 32 ct + l % 32, K rows 16 ks + 8 (l / 32)
// .. +7, which is exactly one packed word.
//
// Consumers. Read A fragments (token rows stored K-step-major, 32 bytes per
// row and K step, the two 16-byte halves swapped on rows whose bit 3 is set,
// so that the 16 lanes the LDS serves together hit distinct banks) and B
// fragments from LDS, and issue v_mfma_f32_32x32x16_bf16 only. With three
// or four occupied 32-row groups the eight consumers split the tile two
// (row halves) by four (64-column quarters); with one or two, eight ways by
// 32 columns.
//
// Hand-over. No workgroup barrier in the main loop: a producer bumps
// full[s % 5] once its part of stage s has landed (its own direct-to-LDS
// load waited by count, its LDS writes waited), and a consumer bumps
// released[s % 5] once its reads of stage s have returned. Nine token-row
// buffers and five weight buffers: producers may run four stages ahead of
// the consumers, and token rows load four stages ahead of the
// dequantisation, across item boundaries, so the next item's first stages
// load while consumers store the current one; both buffers a producer
// refills at stage t were last used by stage t - 5. Row tables (output row
// per tile row, occupied groups) rotate over three slots, one per item in
// flight. Every wait is bounded: past its budget a wave stops waiting, so a
// fault in the hand-over would show as wrong output, never as a hang.
// Outputs are stored straight from the accumulators, two columns per lane
// (adjacent lanes swap values so that each stores 4 bytes of one row).
// ---------------------------------------------------------------------------
constexpr int kPcLead = 4;                        // stages producers may run ahead
constexpr int kPcAhead = 4;                       // token rows load this many stages ahead
constexpr int kPcNB = kPcLead + 1;                // dequantised-weight stage buffers
constexpr int kPcNA = kPcAhead + kPcLead + 1;     // token-row stage buffers
constexpr int kPcTabs = 3;                        // row-table slots (items in flight)
constexpr int kPcSK = 32;                         // K elements per stage
constexpr int kPcKS = kPcSK / 16;                 // 16-wide K steps per stage
constexpr int kPcQ = kChunkK / kPcSK;             // stages per 128-wide packed chunk
constexpr int kPcProd = 8;                        // producer waves
constexpr int kPcCons = 8;                        // consumer waves
constexpr int kPcThreads = 64 * (kPcProd + kPcCons);
constexpr int kPcRowBytes = kPcSK * 2;            // a token row's stage: 64 B
constexpr int kPcAStep = kLmBM * 32;              // one K step of the tile: 4 KiB
constexpr int kPcAStage = kPcKS * kPcAStep;       // 8 KiB: [2 K steps][128 rows][32 B]
constexpr int kPcBStep = 64 * 16;                 // one B fragment: 1 KiB
constexpr int kPcBTile = kPcKS * kPcBStep;        // a 32-column tile's stage: 2 KiB
constexpr int kPcBStage = (kLmBN / 32) * kPcBTile; // 16 KiB
constexpr int kPcSpinBudget = 1 << 24;            // sleeps per wave (s_sleep 1: ~64 cycles)

// Loads each producer issues per stage: one direct-to-LDS row load (for the
// stage kPcAhead ahead), and on the first stage of each chunk the weights of
// the chunk two ahead (two weight and two scale loads). At the signal of
// stage t the loads issued after A(t) are the next kPcAhead row loads and
// the chunks issued at stages t - kPcAhead .. t: two when t starts a chunk,
// else one.
constexpr int kPcALoads = 1;
constexpr int kPcWLoads = 4;
constexpr int kPcSigWait0 = kPcAhead * kPcALoads + 2 * kPcWLoads;       // 12
constexpr int kPcSigWait = kPcAhead * kPcALoads + kPcWLoads;            // 8
// Loads issued after W(c) when stage kPcQ c dequantises it: eight row loads
// and two chunks in steady state; fewer for chunks 0 and 1 (the prologue
// issues them with fewer loads behind them).
constexpr int kPcDeqWait = 2 * kPcQ * kPcALoads + 2 * kPcWLoads;         // 16
constexpr int kPcDeqWait0 = kPcALoads + 2 * kPcWLoads;                   // 9
constexpr int kPcDeqWait1 = (kPcQ + 1) * kPcALoads + 2 * kPcWLoads;      // 13

__device__ __forceinline__ void wait_lgkm0() {
  // s_waitcnt lgkmcnt(0), vector-memory and export counts unconstrained
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// The hand-over counters are read and bumped with inline-asm LDS operations
// (the read waits for itself in the same asm block). As compiler-visible
// LDS accesses they would be ordered behind every outstanding direct-to-LDS
// load (the compiler cannot tell the counters from the load destinations)
// and drain the producers' prefetch queue at every stage. `budget` is the
// wave's remaining sleeps over the whole kernel: once spent, waits return
// at once, so a broken hand-over ends the kernel in about a second instead
// of hanging it.
__device__ __forceinline__ void pc_wait(const int32_t* flag, int target, int& budget) {
  const uint32_t addr = lds_addr(flag);
  for (;;) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    if (__builtin_amdgcn_readfirstlane(v) >= target || budget <= 0) break;
    --budget;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

// One increment per wave; the caller has waited for the data it publishes.
__device__ __forceinline__ void pc_signal(int32_t* flag, int lane) {
  const uint32_t addr = lds_addr(flag);
  const int one = 1;
  asm volatile("" ::: "memory");
  if (lane == 0) asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(one) : "memory");
  asm volatile("" ::: "memory");
}

// Items of one workgroup: tiles x, x + 8, ... of the routed tiles, each
// with its column blocks, every GX-th item from `slot`.
struct PcWalk {
  int x, slot, GX, n_my, nblocks;
  __device__ __forceinline__ void item(const GemmParams& p, int i, int& tile, int& nb,
                                       int& e) const {
    const int q = slot + i * GX;
    const int j = q / nblocks;
    nb = q - j * nblocks;
    tile = x + 8 * j;
    e = tile_expert(p, tile);
  }
};

__device__ __forceinline__ PcWalk pc_walk(const GemmParams& p) {
  PcWalk w;
  const int G = (int)gridDim.x;
  w.x = (int)blockIdx.x & 7;
  w.slot = (int)blockIdx.x >> 3;
  w.GX = G >> 3;
  w.nblocks = p.nblocks;
  const int ntiles = p.mode == 0 ? min(*p.ntp / p.BM, p.num_tiles) : p.num_tiles;
  const int nt_x = ntiles > w.x ? (ntiles - w.x + 7) / 8 : 0;
  const int nq = nt_x * p.nblocks;
  w.n_my = nq > w.slot ? (nq - w.slot + w.GX - 1) / w.GX : 0;
  return w;
}

struct PcLds {
  uint8_t* a;          // [kPcNA][kPcAStage]
  uint8_t* b;          // [kPcNB][kPcBStage]
  int32_t* out;        // [kPcTabs][kLmBM] output row per tile row (-1: none)
  int32_t* gv;         // [kPcTabs][4] 32-row group holds a token
  int32_t* full;       // [kPcNB] producers done with the stage
  int32_t* released;   // [kPcNB] consumers done with the stage
  int32_t* done;       // items whose outputs every consumer has stored
};

// 16-byte half h of row r's 32 bytes of a K step sits at half h ^ (bit 3 of r)
__device__ __forceinline__ int pc_half(int row, int h) { return h ^ ((row >> 3) & 1); }

__device__ __forceinline__ void pc_producer(const GemmParams& p, const PcWalk& wk, const PcLds& s, int pw,
                            int lane) {
  const int KC = p.KC, KS = kPcQ * KC;
  const int S = wk.n_my * KS;                      // stages of this workgroup
  const int U = wk.n_my * KC;                      // chunks
  const uint32_t tile_bytes = (uint32_t)KC * kWBlockBytes;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(uniform_ptr(p.a), p.a_bytes);
  const int c16 = lane & 15;
  const int aks = pw & 1;                          // this producer's K step of token rows
  const int arow0 = (pw >> 1) * 32;                // and its 32 rows
  int budget = kPcSpinBudget;

  // token rows of the item the row loads are on
  uint32_t voff_a[kPcALoads];
  auto enter_item = [&](int i) __attribute__((always_inline)) {
    int tile, nb, e;
    wk.item(p, i, tile, nb, e);
    const int tslot = i % kPcTabs;
    // the row table slot was last read by the epilogue of item i - kPcTabs
    if (i >= kPcTabs) pc_wait(s.done, (i - kPcTabs + 1) * kPcCons, budget);
    const int row = arow0 + (lane & 31);
    RowInfo ri = row_info(p, tile, e, row);
    ri.valid = ri.valid && e >= 0;
    if (aks == 0) {
      if (lane < 32) s.out[tslot * kLmBM + row] = ri.valid ? ri.out_row : -1;
      const uint64_t any = __ballot(lane < 32 && ri.valid);
      if (lane == 0) s.gv[tslot * 4 + (pw >> 1)] = any != 0 ? 1 : 0;
    }
    // lane L: row arow0 + L/2, LDS half L % 2, which holds K half
    // (L % 2) ^ (bit 3 of the row) of K step aks
    const int ar = __shfl(ri.valid ? ri.a_row : -1, lane >> 1, 64);
    const int kh = pc_half(lane >> 1, lane & 1);
    voff_a[0] = ar >= 0 ? (uint32_t)ar * (uint32_t)p.K * 2u + (uint32_t)(aks * 32 + kh * 16)
                        : 0x80000000u;
  };
  // direct-to-LDS loads of stage t's token rows (past the end: the last
  // stage again, into a buffer no consumer reads afterwards)
  auto load_a = [&](int t) __attribute__((always_inline)) {
    const int tt = min(t, S - 1);
    const int i = tt / KS, st = tt - i * KS;
    if (st == 0 && t < S) enter_item(i);
    uint8_t* dst = s.a + (t % kPcNA) * kPcAStage + aks * kPcAStep + arow0 * 32;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)dst, 16,
                                             (int)voff_a[0], st * kPcRowBytes, 0, 0);
  };

  // weights: ring of three chunks of this producer's two 16-column tiles
  u32x4 wv[3][2];
  u32x2 sv[3][2];
  int w_item = -1, wt0 = 0;
  const uint8_t* wbase = p.wpk;
  const uint8_t* sbase = p.spk;
  auto load_w = [&](auto ring_c, int u) __attribute__((always_inline)) {
    constexpr int r = decltype(ring_c)::value;
    u = min(u, U - 1);
    const int i = u / KC, c = u - i * KC;
    if (i != w_item) {
      int tile, nb, e;
      wk.item(p, i, tile, nb, e);
      const size_t ex = (size_t)max(e, 0) * p.NT;
      wbase = p.wpk + ex * tile_bytes;
      sbase = p.spk + ex * (size_t)KC * kSBlockBytes;
      wt0 = nb * (kLmBN / 16) + pw * 2;
      w_item = i;
    }
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(uniform_ptr(wbase), (uint32_t)p.NT * tile_bytes);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(uniform_ptr(sbase), (uint32_t)p.NT * KC * kSBlockBytes);
    const TileAddr wa = tile_addr(p, wt0, kWBlockBytes), sa = tile_addr(p, wt0, kSBlockBytes);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      wv[r][t] = __builtin_amdgcn_raw_buffer_load_b128(rw, lane * 16,
                                                       wa.base + t * wa.tile + c * wa.chunk,
                                                       kNonTemporal);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      sv[r][t] = __builtin_amdgcn_raw_buffer_load_b64(rs, c16 * 8,
                                                      sa.base + t * sa.tile + c * sa.chunk, 0);
  };
  // dequantise quarter j (word j, scale group j) of the chunk in ring slot
  // r into weight buffer b: this producer's 32-column tile ct = pw, K step
  // lane / 32 of the stage
  const uint32_t bdst0 = (uint32_t)(pw * kPcBTile) +
                         (uint32_t)((c16 + 32 * ((lane >> 4) & 1)) * 16 + (lane >> 5) * kPcBStep);
  auto dequant = [&](auto ring_c, auto j_c, int b) __attribute__((always_inline)) {
    constexpr int r = decltype(ring_c)::value;
    constexpr int j = decltype(j_c)::value;
    uint8_t* dst = s.b + b * kPcBStage + bdst0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t sw = sv[r][t][j >> 1];      // scales of groups 2 (j/2), +1
      const float sc = (j & 1) ? bf16_hi(sw) : bf16_lo(sw);
      const u32x4 v = dequant8(wv[r][t][j], sc, -8.0f * sc);
      *(u32x4*)(dst + t * 256) = v;
    }
  };

  if (S == 0) return;
  // Prologue: the token rows of the first kPcAhead stages (with item 0's
  // row table), then two weight chunks.
#pragma unroll
  for (int t = 0; t < kPcAhead; ++t) load_a(t);
  load_w(std::integral_constant<int, 0>{}, 0);
  load_w(std::integral_constant<int, 1>{}, 1);

  // Step t: [stage t - kPcNB released: both buffers refilled below are
  // free] A(t + kPcAhead) [W(t/4 + 2) when t starts a chunk] [W(t/4) has
  // landed] dequantise B(t) [A(t) has landed] signal full(t). Steps are
  // unrolled in groups of 12 (three chunks), so the register ring slot of
  // every chunk is a constant.
  auto step = [&](int t, auto k_c, auto deq_wait_c) __attribute__((always_inline)) {
    constexpr int k = decltype(k_c)::value;          // t % 12
    constexpr int deq_wait = decltype(deq_wait_c)::value;
    constexpr int ring = k / kPcQ;                   // chunk t/4 lives in ring (t/4) % 3
    if (t >= kPcNB) pc_wait(&s.released[t % kPcNB], (t / kPcNB) * kPcCons, budget);
    load_a(t + kPcAhead);
    if constexpr (k % kPcQ == 0) {
      load_w(std::integral_constant<int, (ring + 2) % 3>{}, t / kPcQ + 2);
      wait_vmcnt<deq_wait>();
    }
    dequant(std::integral_constant<int, ring>{}, std::integral_constant<int, k % kPcQ>{},
            t % kPcNB);
    wait_vmcnt<(k % kPcQ == 0) ? kPcSigWait0 : kPcSigWait>();
    wait_lgkm0();
    pc_signal(&s.full[t % kPcNB], lane);
  };
  auto group = [&](int t0, auto first_c) __attribute__((always_inline)) {
    constexpr bool first = decltype(first_c)::value;
    using WS = std::integral_constant<int, kPcDeqWait>;
    static_for<12>([&](auto k_c) __attribute__((always_inline)) {
      constexpr int k = decltype(k_c)::value;
      constexpr int dw = !first ? kPcDeqWait : (k == 0 ? kPcDeqWait0 : (k == 4 ? kPcDeqWait1 : kPcDeqWait));
      if (t0 + k < S) step(t0 + k, k_c, std::integral_constant<int, dw>{});
      __builtin_amdgcn_sched_barrier(0);
      (void)WS{};
    });
  };
  group(0, std::true_type{});
  for (int t0 = 12; t0 < S; t0 += 12) group(t0, std::false_type{});
  // every direct-to-LDS load has landed before the workgroup can end
  wait_vmcnt<0>();
}

template <int NV, int NT>
__device__ __forceinline__ void pc_store(const GemmParams& p, const int32_t* out_rows, int nb,
                                         int gr0, int ct0, int lane, const f32x16 (&acc)[2][2]) {
  const int l32 = lane & 31, kq = lane >> 5;
  const bool odd = lane & 1;
#pragma unroll
  for (int m = 0; m < NV; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // output rows of accumulator elements 4i .. 4i+3: rows R0 .. R0+3
      const int R0 = (gr0 + m) * 32 + 8 * i + 4 * kq;
      const int4 orow4 = *(const int4*)(out_rows + R0);
      const int ov[4] = {orow4.x, orow4.y, orow4.z, orow4.w};
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const int C = (ct0 + n) * 32 + l32;                   // column in the block
          float x0 = acc[m][n][4 * i + r], x1 = acc[m][n][4 * i + r + 1];
          const int o0 = ov[r], o1 = ov[r + 1];
          if (p.mode == 0 && p.topk_w) {
            x0 *= o0 >= 0 ? p.topk_w[o0] : 1.0f;
            x1 *= o1 >= 0 ? p.topk_w[o1] : 1.0f;
          }
          // even lane stores (R; C, C+1), odd lane (R+1; C-1, C)
          const float send = odd ? x0 : x1;
          const float recv = __int_as_float(
              __builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
          const float lo = odd ? recv : x0, hi = odd ? x1 : recv;
          const int orow = odd ? o1 : o0;
          const int col = nb * kLmBN + (odd ? C - 1 : C);
          const uint32_t v = cvt_pk_bf16(lo, hi);
          if (orow >= 0) *(uint32_t*)(p.c + (size_t)orow * p.N + col) = v;
        }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// All stages of one item and its stores, for a consumer whose tile is NV
// 32-row groups from gr0 by NT 32-column tiles from ct0 (NV = 0: the item
// has no token; stages are only waited for and released). t is the
// workgroup's stage counter at the item's first stage. Fragment reads run
// one K step ahead of the MFMAs, also across stages: stage t is released
// as soon as its reads have returned, and before its last K step's MFMAs
// the consumer waits for stage t + 1 and reads its first fragments, so both
// latencies hide behind MFMAs already issued.
template <int NV, int NT>
__device__ __forceinline__ void pc_consume_item(const GemmParams& p, const PcLds& s, int lane,
                                                int t, int KS, int nb, int gr0, int ct0,
                                                const int32_t* orows, int& budget) {
  if constexpr (NV == 0) {
    for (int st = 0; st < KS; ++st, ++t) {
      pc_wait(&s.full[t % kPcNB], (t / kPcNB + 1) * kPcProd, budget);
      pc_signal(&s.released[t % kPcNB], lane);
    }
  } else {
    f32x16 acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[m][n] = f32x16{};
    // lane's A fragment: row gr0*32 + lane % 32, K half lane / 32 of the K
    // step; B fragment: tile ct0, lane's 16 bytes. Every other fragment is at
    // a constant offset from these.
    const int arow = gr0 * 32 + (lane & 31);
    const uint8_t* a0 = s.a + arow * 32 + pc_half(arow, lane >> 5) * 16;
    const uint8_t* b0 = s.b + ct0 * kPcBTile + lane * 16;
    u32x4 av[2][NV], bv[2][NT];
    auto rd = [&](int slot, int tt, int ks) __attribute__((always_inline)) {
      const uint8_t* ab = a0 + (tt % kPcNA) * kPcAStage + ks * kPcAStep;
      const uint8_t* bb = b0 + (tt % kPcNB) * kPcBStage + ks * kPcBStep;
#pragma unroll
      for (int m = 0; m < NV; ++m) av[slot][m] = *(const u32x4*)(ab + m * 32 * 32);
#pragma unroll
      for (int n = 0; n < NT; ++n) bv[slot][n] = *(const u32x4*)(bb + n * kPcBTile);
    };
    auto mma = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < NV; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = mfma32(av[slot][m], bv[slot][n], acc[m][n]);
    };
    pc_wait(&s.full[t % kPcNB], (t / kPcNB + 1) * kPcProd, budget);
    rd(0, t, 0);
    for (int st = 0; st < KS; ++st, ++t) {
      rd(1, t, 1);
      mma(0);
      // the reads of stage t have returned once the last one has
      wait_lgkm0();
      pc_signal(&s.released[t % kPcNB], lane);
      if (st + 1 < KS) {
        pc_wait(&s.full[(t + 1) % kPcNB], ((t + 1) / kPcNB + 1) * kPcProd, budget);
        rd(0, t + 1, 0);
      }
      mma(1);
    }
    pc_store<NV, NT>(p, orows, nb, gr0, ct0, lane, acc);
  }
}

__device__ __forceinline__ void pc_consumer(const GemmParams& p, const PcWalk& wk, const PcLds& s, int cw,
                            int lane) {
  const int KS = kPcQ * p.KC;
  int budget = kPcSpinBudget;
  for (int i = 0, t = 0; i < wk.n_my; ++i, t += KS) {
    int tile, nb, e;
    wk.item(p, i, tile, nb, e);
    const int tslot = i % kPcTabs;
    // the item's row table is published with its first stage
    pc_wait(&s.full[t % kPcNB], (t / kPcNB + 1) * kPcProd, budget);
    const int* gv = s.gv + tslot * 4;
    // occupied 32-row groups: one past the last group holding a token
    const int g = __builtin_amdgcn_readfirstlane(gv[3] ? 4 : gv[2] ? 3 : gv[1] ? 2 : gv[0] ? 1 : 0);
    const int32_t* orows = s.out + tslot * kLmBM;
    if (g >= 3) {
      // two row halves x four 64-column quarters
      const int gr0 = 2 * (cw >> 2), ct0 = 2 * (cw & 3);
      if (g - gr0 >= 2)
        pc_consume_item<2, 2>(p, s, lane, t, KS, nb, gr0, ct0, orows, budget);
      else
        pc_consume_item<1, 2>(p, s, lane, t, KS, nb, gr0, ct0, orows, budget);
    } else if (g == 2) {
      // eight 32-column slices over both groups
      pc_consume_item<2, 1>(p, s, lane, t, KS, nb, 0, cw, orows, budget);
    } else if (g == 1) {
      pc_consume_item<1, 1>(p, s, lane, t, KS, nb, 0, cw, orows, budget);
    } else {
      pc_consume_item<0, 1>(p, s, lane, t, KS, nb, 0, 0, orows, budget);
    }
    // this consumer no longer reads item i's row table
    wait_lgkm0();
    pc_signal(s.done, lane);
  }
}

__global__ __launch_bounds__(kPcThreads, 1) void gemm_large_m_pc_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_a[kPcNA * kPcAStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s_b[kPcNB * kPcBStage];
  __shared__ __attribute__((aligned(16))) int32_t s_out[kPcTabs * kLmBM];
  __shared__ int32_t s_gv[kPcTabs * 4];
  __shared__ int32_t s_full[kPcNB];
  __shared__ int32_t s_released[kPcNB];
  __shared__ int32_t s_done;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (threadIdx.x < kPcNB) {
    s_full[threadIdx.x] = 0;
    s_released[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) s_done = 0;
  __syncthreads();
  const PcWalk wk = pc_walk(p);
  if (wk.n_my == 0) return;
  // (an offset the compiler cannot fold keeps this a run-time value: as a
  // constant it would become a global whose initializer holds LDS
  // addresses, which the target cannot emit)
  int z = 0;
  asm volatile("" : "+s"(z));
  const PcLds s{s_a + z, s_b + z, s_out + z, s_gv + z, s_full + z, s_released + z, &s_done + z};
  // waves 0..7 consume, 8..15 produce: each SIMD holds two of each
  if (w >= kPcCons)
    pc_producer(p, wk, s, w - kPcCons, lane);
  else
    pc_consumer(p, wk, s, w, lane);
}

template <int TM, int NTW, int WK, int D>
static int launch_small_m_inst(const GemmParams& gp, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((gemm_small_m_kernel<TM, NTW, WK, D>), dim3(grid), dim3(256), 0, st, gp);
  return (int)hipGetLastError();
}

template <int TM, int NTW, int WK>
static int launch_small_m_depth(const GemmParams& gp, unsigned grid, hipStream_t st, int depth) {
  constexpr int D0 = small_m_depth(TM, NTW);
  if constexpr (TM == 1 && NTW == 4) {
    // depth 4 would need more than 256 VGPRs and spill
    if (depth == 2) return launch_small_m_inst<TM, NTW, WK, 2>(gp, grid, st);
    if (depth == 3) return launch_small_m_inst<TM, NTW, WK, 3>(gp, grid, st);
  }
  return launch_small_m_inst<TM, NTW, WK, D0>(gp, grid, st);
}

template <int TM, int NTW>
static int launch_small_m_wk(const GemmParams& gp, unsigned grid, hipStream_t st, int wk,
                             int depth) {
  if constexpr (small_m_wave_rows(TM, NTW, 1))
    if (wk == 1) return launch_small_m_depth<TM, NTW, 1>(gp, grid, st, depth);
  if (wk == 2) return launch_small_m_depth<TM, NTW, 2>(gp, grid, st, depth);
  if (wk == 4) return launch_small_m_depth<TM, NTW, 4>(gp, grid, st, depth);
  return (int)hipErrorInvalidConfiguration;
}

// Gang schedule: one workgroup of kGangGroups groups per CU. The launch asks
// for enough LDS that a second workgroup never fits beside the first, so
// every CU runs its groups in lock-step to the end.
template <int TM, int NTW>
static int launch_xs_gang(const GemmParams& gp, int64_t items, hipStream_t st) {
  constexpr int S = kGangGroups;
  constexpr size_t stat = (size_t)S * xs_gang_stride<TM, 2>();
  constexpr size_t one_per_cu = kLdsPerCU / 2 + 1024;
  const size_t dyn = stat < one_per_cu ? one_per_cu - stat : 0;
  const int64_t need = (items + 8 * S - 1) / (8 * S) * 8;
  const unsigned grid = (unsigned)std::min<int64_t>(kNumCUs, need);
  hipLaunchKernelGGL((gemm_small_m_xs_gang_kernel<TM, NTW, 2, S>), dim3(grid), dim3(256 * S),
                     dyn, st, gp);
  return (int)hipGetLastError();
}

// Stream-K gang: one workgroup per CU (the launch asks for more than half a
// CU's LDS), S groups of four waves. The kernel keeps a group's items
// within two token tiles; the caller checks that bound for the call.
template <int TM, int NTW, int S>
static int launch_sk(const GemmParams& gp, hipStream_t st) {
  constexpr size_t stat = (size_t)S * sk_group_bytes<TM, NTW>();
  static_assert(stat <= (size_t)kLdsPerCU, "stream-K groups exceed a CU's LDS");
  constexpr size_t one_per_cu = kLdsPerCU / 2 + 1024;
  const size_t dyn = stat < one_per_cu ? one_per_cu - stat : 0;
  hipLaunchKernelGGL((gemm_small_m_sk_kernel<TM, NTW, S>), dim3((unsigned)kNumCUs),
                     dim3(256 * S), dyn, st, gp);
  return (int)hipGetLastError();
}

// Token tiles the plan expects (its estimate, est_tiles / column blocks).
static int64_t plan_tiles_m(const qma_plan_t& pl) {
  const int64_t nb = pl.block_n > 0 ? pl.n / pl.block_n : 0;
  return nb > 0 ? pl.est_tiles / nb : 0;
}

int launch_gemm(const GemmArgs& g, void* stream) {
  const Layer& L = *g.layer;
  const qma_plan_t& pl = *g.plan;
  hipStream_t st = (hipStream_t)stream;
  GemmParams gp{};
  gp.a = g.a;
  gp.wpk = (const uint8_t*)g.packed;
  gp.spk = (const uint8_t*)g.packed + L.w_bytes;
  gp.c = g.c;
  gp.ws = (float*)g.ws;
  gp.sorted_ids = g.sorted_ids;
  gp.expert_ids = g.expert_ids;
  gp.ntp = g.ntp;
  gp.topk_w = g.topk_weights;
  gp.m_indices = g.m_indices;
  gp.masked_m = g.masked_m;
  gp.a_bytes = (uint32_t)g.a_bytes;
  gp.mode = g.mode;
  gp.a_row_div = g.a_row_div;
  gp.num_tiles = g.num_tiles;
  gp.nblocks = L.N / pl.block_n;
  gp.split = pl.split_k;
  gp.num_slots = g.num_slots;
  gp.Mb = g.Mb;
  gp.tiles_per_expert = g.tiles_per_expert;
  gp.rows_cap = g.rows_cap;
  gp.cap = g.sorted_cap;
  gp.E = L.E;
  gp.N = L.N;
  gp.K = L.K;
  gp.NT = (int32_t)L.n_tiles;
  gp.KC = (int32_t)L.k_chunks;
  gp.BM = pl.block_m;
  gp.wg_log2 = L.wg_log2;
  gp.act = L.act;
  gp.fold = 1;
  const int64_t tiles_pad = (g.num_tiles + 7) / 8 * 8;
  const int64_t grid = tiles_pad * gp.nblocks * gp.split;
  if (grid <= 0) return 0;
  if (grid >= (1ll << 24)) return (int)hipErrorInvalidConfiguration;
  if (pl.kernel == QMA_KERNEL_LARGE_M_PC) {
    if (pl.block_m != kLmBM || pl.block_n != kLmBN || L.N % kLmBN != 0 || gp.split != 1)
      return (int)hipErrorInvalidConfiguration;
    // persistent: one workgroup per CU, a multiple of the 8 XCDs
    hipLaunchKernelGGL(gemm_large_m_pc_kernel, dim3((unsigned)kNumCUs), dim3(kPcThreads), 0, st,
                       gp);
    return (int)hipGetLastError();
  }
  if (pl.kernel == QMA_KERNEL_LARGE_M) {
    if (pl.block_m != kLmBM || pl.block_n != kLmBN || L.N % kLmBN != 0)
      return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gemm_large_m_kernel, dim3((unsigned)grid), dim3(256), 0, st, gp);
    int err = (int)hipGetLastError();
    if (err == 0 && gp.split > 1) {
      const int64_t total = (int64_t)gp.num_tiles * gp.BM * (gp.N / 4);
      const unsigned rb = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
      hipLaunchKernelGGL(splitk_reduce_kernel, dim3(rb), dim3(256), 0, st, gp);
      err = (int)hipGetLastError();
    }
    return err;
  }
  const int tm = pl.block_m / 16;
  const int wk = pl.waves_k;
  const int ntw = pl.block_n / (16 * (4 / std::max(wk, 1)));
  const int depth = pl.k_depth / kChunkK;
  const bool xs = small_m_shared_rows(tm, ntw, wk) && ntw * 64 == pl.block_n && pl.n_stream == 1;
  if (pl.schedule == QMA_SCHEDULE_DYNAMIC) {
    if (!xs || tm > 2 || gp.split != 1 || g.ws == nullptr)
      return (int)hipErrorInvalidConfiguration;
    gp.nstream = 1;
    gp.nbtot = gp.nblocks;
    gp.work = (int32_t*)g.ws;
    hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(64), 0, st, gp.work);
    const dim3 dg((unsigned)(3 * kNumCUs));
    if (tm == 1 && ntw == 4)
      hipLaunchKernelGGL((gemm_small_m_xs_dyn_kernel<1, 4, 2>), dg, dim3(256), 0, st, gp);
    else if (tm == 1)
      hipLaunchKernelGGL((gemm_small_m_xs_dyn_kernel<1, 2, 2>), dg, dim3(256), 0, st, gp);
    else if (ntw == 4)
      hipLaunchKernelGGL((gemm_small_m_xs_dyn_kernel<2, 4, 2>), dg, dim3(256), 0, st, gp);
    else
      hipLaunchKernelGGL((gemm_small_m_xs_dyn_kernel<2, 2, 2>), dg, dim3(256), 0, st, gp);
    return (int)hipGetLastError();
  }
  int err = (int)hipErrorInvalidConfiguration;
  if (pl.n_stream > 1 || xs) {
    // one K partition per workgroup: 16-row tiles streaming column blocks,
    // or 16/32/64-row tiles with the token rows shared through LDS (these
    // also take split-K)
    if (wk != 1 || (ntw != 2 && ntw != 4) || ntw * 64 != pl.block_n ||
        (pl.n_stream > 1 && (tm != 1 || gp.split != 1)))
      return (int)hipErrorInvalidConfiguration;
    gp.nstream = pl.n_stream;
    gp.nbtot = gp.nblocks;
    gp.nblocks = (gp.nbtot + gp.nstream - 1) / gp.nstream;
    gp.fold = xcd_fold(plan_tiles_m(pl), gp.nblocks);
    const int64_t vt_pad = ((int64_t)g.num_tiles * gp.fold + 7) / 8 * 8;
    const dim3 sg((unsigned)(vt_pad * (gp.nblocks / gp.fold) * gp.split));
    if (pl.schedule == QMA_SCHEDULE_STREAM_K) {
      if (!xs || g.mode != 0 || gp.split != 1 || tm > 2 || gp.KC < kStreamChunks ||
          gp.nstream != 1 || !stream_k_fits(g.num_tiles, gp.nblocks, gp.KC, ntw))
        return (int)hipErrorInvalidConfiguration;
      gp.fold = 1;
      if (tm == 1 && ntw == 4)
        err = launch_sk<1, 4, sk_groups(4)>(gp, st);
      else if (tm == 1)
        err = launch_sk<1, 2, sk_groups(2)>(gp, st);
      else if (ntw == 4)
        err = launch_sk<2, 4, sk_groups(4)>(gp, st);
      else
        err = launch_sk<2, 2, sk_groups(2)>(gp, st);
    } else if (pl.schedule == QMA_SCHEDULE_GANG) {
      if (!xs) return (int)hipErrorInvalidConfiguration;
      if (tm == 1 && ntw == 4)
        err = launch_xs_gang<1, 4>(gp, sg.x, st);
      else if (tm == 1)
        err = launch_xs_gang<1, 2>(gp, sg.x, st);
      else if (tm == 2 && ntw == 4)
        err = launch_xs_gang<2, 4>(gp, sg.x, st);
      else if (tm == 2)
        err = launch_xs_gang<2, 2>(gp, sg.x, st);
      else
        err = launch_xs_gang<4, 2>(gp, sg.x, st);
    } else {
      if (xs && tm == 1 && ntw == 4)
        hipLaunchKernelGGL((gemm_small_m_xs_kernel<1, 4, 2>), sg, dim3(256), 0, st, gp);
      else if (xs && tm == 1)
        hipLaunchKernelGGL((gemm_small_m_xs_kernel<1, 2, 2>), sg, dim3(256), 0, st, gp);
      else if (xs && tm == 2 && ntw == 4)
        hipLaunchKernelGGL((gemm_small_m_xs_kernel<2, 4, 2>), sg, dim3(256), 0, st, gp);
      else if (xs && tm == 2)
        hipLaunchKernelGGL((gemm_small_m_xs_kernel<2, 2, 2>), sg, dim3(256), 0, st, gp);
      else if (xs)
        hipLaunchKernelGGL((gemm_small_m_xs_kernel<4, 2, 2>), sg, dim3(256), 0, st, gp);
      else if (ntw == 4 && gp.KC <= 2)
        hipLaunchKernelGGL((gemm_small_m_stream_kernel<4, 2, true>), sg, dim3(256), 0, st, gp);
      else if (ntw == 4)
        hipLaunchKernelGGL((gemm_small_m_stream_kernel<4, 4, false>), sg, dim3(256), 0, st, gp);
      else if (gp.KC <= 2)
        hipLaunchKernelGGL((gemm_small_m_stream_kernel<2, 2, true>), sg, dim3(256), 0, st, gp);
      else
        hipLaunchKernelGGL((gemm_small_m_stream_kernel<2, 4, false>), sg, dim3(256), 0, st, gp);
      err = (int)hipGetLastError();
    }
  } else {
    if (!small_m_wave_rows(tm, ntw, wk) || ntw * 16 * (4 / wk) != pl.block_n)
      return (int)hipErrorInvalidConfiguration;
    gp.fold = xcd_fold(plan_tiles_m(pl), gp.nblocks);
    const int64_t vt_pad = ((int64_t)g.num_tiles * gp.fold + 7) / 8 * 8;
    const unsigned wgrid = (unsigned)(vt_pad * (gp.nblocks / gp.fold) * gp.split);
#define QMA_SMALL_M_CASE(TM_, NTW_) \
  if (tm == TM_ && ntw == NTW_) err = launch_small_m_wk<TM_, NTW_>(gp, wgrid, st, wk, depth);
    QMA_SMALL_M_CASE(1, 1)
    QMA_SMALL_M_CASE(1, 2)
    QMA_SMALL_M_CASE(1, 4)
    QMA_SMALL_M_CASE(2, 1)
    QMA_SMALL_M_CASE(2, 2)
    QMA_SMALL_M_CASE(4, 1)
#undef QMA_SMALL_M_CASE
  }
  if (err != 0) return err;
  if (gp.split > 1) {
    const int64_t total = (int64_t)gp.num_tiles * gp.BM * (gp.N / 4);
    const unsigned rb = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(rb), dim3(256), 0, st, gp);
    err = (int)hipGetLastError();
  }
  return err;
}

// ---------------------------------------------------------------------------
// silu_and_mul: y[r, j] = silu(x[r, j]) * x[r, I + j] in fp32 ([announce]
// measurement section: the activation between gate/up and down).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void silu_mul_vec8_kernel(const uint16_t* __restrict__ x,
                                                            uint16_t* __restrict__ y, int64_t R,
                                                            int32_t I) {
  const int64_t per_row = I / 8;
  const int64_t total = R * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row;
    const int64_t j = (i - r * per_row) * 8;
    const u32x4 g = *(const u32x4*)(x + r * 2 * I + j);
    const u32x4 u = *(const u32x4*)(x + r * 2 * I + I + j);
    u32x4 o;
    o.x = pack_bf16x2(silu_mul(bf16_lo(g.x), bf16_lo(u.x)), silu_mul(bf16_hi(g.x), bf16_hi(u.x)));
    o.y = pack_bf16x2(silu_mul(bf16_lo(g.y), bf16_lo(u.y)), silu_mul(bf16_hi(g.y), bf16_hi(u.y)));
    o.z = pack_bf16x2(silu_mul(bf16_lo(g.z), bf16_lo(u.z)), silu_mul(bf16_hi(g.z), bf16_hi(u.z)));
    o.w = pack_bf16x2(silu_mul(bf16_lo(g.w), bf16_lo(u.w)), silu_mul(bf16_hi(g.w), bf16_hi(u.w)));
    *(u32x4*)(y + r * I + j) = o;
  }
}

__global__ __launch_bounds__(256) void silu_mul_scalar_kernel(const uint16_t* __restrict__ x,
                                                              uint16_t* __restrict__ y, int64_t R,
                                                              int32_t I) {
  const int64_t total = R * I;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / I;
    const int64_t j = i - r * I;
    const float g = __uint_as_float((uint32_t)x[r * 2 * I + j] << 16);
    const float u = __uint_as_float((uint32_t)x[r * 2 * I + I + j] << 16);
    y[i] = (uint16_t)(pack_bf16x2(silu_mul(g, u), 0.f) & 0xFFFFu);
  }
}

int launch_silu_and_mul(const uint16_t* x, uint16_t* y, int64_t R, int32_t I, void* stream) {
  const bool vec = (I % 8 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0);
  const int64_t work = vec ? R * (I / 8) : R * I;
  const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 16384);
  if (vec)
    hipLaunchKernelGGL(silu_mul_vec8_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, x,
                       y, R, I);
  else
    hipLaunchKernelGGL(silu_mul_scalar_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       x, y, R, I);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k combine: out[t, n] = sum_k w[t, k] * c2[t*topk + k, n], fp32 sums in
// k order, slots of experts outside [0, E) skipped when ids are given.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Router: softmax over the E logits of a token and its top-k experts, one
// wave per token with the row in registers (E <= 1024: 16 per lane). The
// choice compares logits (softmax is monotone, so no rounding can reorder
// it), k rounds of a wave argmax over the experts not yet chosen, the
// larger logit winning and the lower index on a tie.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool router_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          int T, int E, int topk,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  constexpr int PER = 16;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[PER];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -__builtin_huge_valf();
    m = fmaxf(m, v[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i < E) sum += expf(v[i] - m);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  uint32_t taken = 0;  // bit i: expert lane + 64 i already chosen
  for (int k = 0; k < topk; ++k) {
    float bv = -__builtin_huge_valf();
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && router_better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (router_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      ids[(size_t)t * topk + k] = bi;
      if (w) w[(size_t)t * topk + k] = expf(bv - m) / sum;
    }
  }
}

int launch_router_topk(const float* logits, int32_t T, int32_t E, int32_t topk, int32_t* ids,
                       float* w, void* stream) {
  hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0,
                     (hipStream_t)stream, logits, T, E, topk, ids, w);
  return (int)hipGetLastError();
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ c2,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ ids,
                                                      int32_t E, int32_t T, int32_t topk,
                                                      int32_t N, uint16_t* __restrict__ out) {
  const int64_t total = (int64_t)T * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / N;
    const int64_t n = i - t * N;
    float s = 0.f;
    for (int k = 0; k < topk; ++k) {
      const int64_t slot = t * topk + k;
      if (ids && (unsigned)ids[slot] >= (unsigned)E) continue;
      s = __builtin_fmaf(w[slot], __uint_as_float((uint32_t)c2[slot * N + n] << 16), s);
    }
    out[i] = (uint16_t)(pack_bf16x2(s, 0.f) & 0xFFFFu);
  }
}

int launch_combine(const uint16_t* c2, const float* w, const int32_t* ids, int32_t E, int32_t T,
                   int32_t topk, int32_t N, uint16_t* out, void* stream) {
  const int64_t total = (int64_t)T * N;
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 16384);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, c2, w,
                     ids, E, T, topk, N, out);
  return (int)hipGetLastError();
}

}  // namespace qma
