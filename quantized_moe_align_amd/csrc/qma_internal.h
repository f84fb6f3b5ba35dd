// Internal declarations shared by the host layer (qma_host.cpp) and the
// kernels (qma_kernels.hip). Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/qma.h"

// Packed layout (fixed at load). For expert e, 16-row tile nt, and 128-wide
// K chunk kc, one 1 KiB block holds the uint4 values in MFMA fragment order:
// lane l (0..63) owns 16 bytes = 4 words; word j covers row nt*16 + l%16,
// K range kc*128 + j*32 + (l/16)*8 .. +7. Inside a word the eight values sit
// in the order (k0, k4, k1, k5, k2, k6, k3, k7) from the low nibble up, so
// that w & 0x0F0F0F0F holds k0..k3 and (w >> 4) & 0x0F0F0F0F holds k4..k7,
// one value per byte. A second region holds the scales: per (e, nt, kc) 128 bytes
// laid out [16 rows][4 groups] bf16.
// Block order inside an expert: tiles are taken G = 1 << wg_log2 at a time;
// a group's K chunks follow each other, and within one chunk the group's G
// tiles sit side by side. Block (nt, kc) is therefore number
// ((nt / G) * KC + kc) * G + nt % G of the expert (weights and scales alike).
// G = 1 (tile-major: each tile's chunks contiguous) for most layers; G = 16
// for gate_up projections whose N is a multiple of 256, where a 256-column
// workgroup then streams one contiguous 16 KiB run per K chunk (measured
// 2-3 % faster on the EP8 decode gate_up share; down projections ran 4-7 %
// slower that way, so they keep G = 1).
namespace qma {

constexpr int kTileN = 16;       // weight rows per MFMA tile
constexpr int kChunkK = 128;     // K elements per packed chunk
constexpr int kGroup = 32;       // K elements per scale
constexpr int kWBlockBytes = 1024;
constexpr int kSBlockBytes = 128;
constexpr int kMaxExperts = 1024;  // moe_align's single-workgroup limit
constexpr int kNumCUs = 256;
// K is short (fewer chunks than this) when a small-M workgroup would see too
// few chunks to fill its load pipeline
constexpr int kStreamChunks = 8;
// chunks a streaming small-M workgroup walks in all (column blocks x K
// chunks). On the TP8 down share (K = 256, two chunks per block) 14 chunks
// (7 blocks) ran 3-4 % faster than 8 and 28.
constexpr int kStreamTargetChunks = 14;
// fewest 128-wide K chunks a small-M split-K partition is planned with: a
// shorter run pays the pipeline's start and the reduction for too little
// streaming
constexpr int kSplitChunks = 14;
constexpr int kLdsPerCU = 160 * 1024;
// Small-M launches deal token tiles to the 8 XCDs in turn, all column blocks
// of a tile on one XCD, so that its rows stay in that XCD's L2. With few
// tiles that leaves XCDs idle or uneven (an EP128 share: 3 tiles on 3 of
// the 8 XCDs). The fold splits each tile's column blocks into f groups
// dealt as separate tiles (each XCD then reads the rows of the tiles it
// holds): the smallest f in {1, 2, 4, 8} dividing nblocks whose t * f
// virtual tiles fill the 8 XCDs to within 10 % of even.
inline int xcd_fold(int64_t tiles, int64_t nblocks) {
  if (tiles <= 0) return 1;
  for (int f = 1; f <= 8; f *= 2) {
    if (nblocks % f != 0) break;
    const int64_t v = tiles * f;
    if ((v + 7) / 8 * 8 * 10 <= v * 11) return f;
  }
  int f = 8;
  while (f > 1 && nblocks % f != 0) f /= 2;
  return f;
}

// Gang schedule: four-wave groups per workgroup, one workgroup per CU. The
// planner takes it for a shared-row GEMM whose planned items fill between
// kGangMinFill sixths and all of one round of kGangGroups * kNumCUs slots.
constexpr int kGangGroups = 3;
constexpr int kGangMinFill = 5;
// bytes at the end of the workspace holding a dynamic schedule's counter
constexpr int kWorkCounterBytes = 256;
// size of the library's static device scratch (qma_indexed_gemm_scratch):
// the split-K partials and the work counter of one call
constexpr size_t kScratchBytes = (size_t)32 << 20;

struct Layer {
  int32_t E, N, K;
  int32_t path;
  int32_t profile;
  int32_t wg_log2;     // log2 of the tiles per block group (packed layout)
  int32_t act;         // 1: gate_up layer with silu(gate) * up fused (packed tiles interleaved)
  int64_t n_tiles;     // N / 16
  int64_t k_chunks;    // K / 128
  size_t w_bytes;      // weight region
  size_t s_bytes;      // scale region
};

// log2 of the tile group of a gate_up projection whose N is a multiple of 256
constexpr int kGateUpGroupLog2 = 4;

// Arguments the GEMM launchers take, after host validation.
struct GemmArgs {
  const Layer* layer;
  const qma_plan_t* plan;
  const uint16_t* a;
  const void* packed;
  uint16_t* c;
  void* ws;
  // row mapping
  int32_t mode;              // 0 indexed, 1 contiguous, 2 masked
  int32_t a_row_div;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntp;
  int32_t num_tiles;         // token tiles in the grid (before padding)
  int32_t num_slots;
  const float* topk_weights;
  const int32_t* m_indices;
  const int32_t* masked_m;
  int32_t Mb;                // masked budget
  int32_t tiles_per_expert;  // masked
  int32_t rows_cap;          // rows of the split-K workspace
  int32_t sorted_cap;        // entries of sorted_ids (indexed)
  int64_t a_bytes;           // bytes of the activation buffer
};

// Launchers (qma_kernels.hip). Each returns a hipError_t as int.
int launch_moe_align(const int32_t* ids, int32_t R, int32_t E, int32_t B,
                     int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                     int32_t cap, void* stream);
int launch_prepack(const Layer& L, const int32_t* qweight,
                   const uint16_t* scales, void* packed, void* stream);
int launch_silu_and_mul(const uint16_t* x, uint16_t* y, int64_t R, int32_t I,
                        void* stream);
int launch_gemm(const GemmArgs& g, void* stream);

// Groups per stream-K workgroup: four for the 128-column instances (at
// most 128 VGPRs), three for the 256-column ones (at most 168).
constexpr int sk_groups(int ntw) { return ntw == 4 ? 3 : 4; }

// Whether a stream-K launch keeps every group's unit range within two token
// tiles for any routed tile count up to num_tiles: a workgroup holds at
// most ceil(items / CUs) items, a group ceil(that * KC / S) units, and a
// range of L units touches at most 1 + ceil((L - 1) / KC) items.
inline bool stream_k_fits(int64_t num_tiles, int64_t nblocks, int64_t kc, int ntw) {
  const int S = sk_groups(ntw);
  if (num_tiles <= 0 || nblocks <= 0 || kc <= 0) return false;
  const int64_t per_wg = (num_tiles * nblocks + kNumCUs - 1) / kNumCUs;
  if (per_wg * kc >= (1ll << 30)) return false;
  const int64_t per_group = (per_wg * kc + S - 1) / S;
  const int64_t span = 1 + (per_group - 1 + kc - 1) / kc;
  return span - 1 <= nblocks;
}
int launch_router_topk(const float* logits, int32_t T, int32_t E, int32_t topk,
                       int32_t* ids, float* w, void* stream);
int launch_combine(const uint16_t* c2, const float* w, const int32_t* ids,
                   int32_t E, int32_t T, int32_t topk, int32_t N,
                   uint16_t* out, void* stream);
// Device address of the static scratch on the current device (looked up once
// per device); returns a hipError_t as int.
int scratch_device_ptr(void** out);

}  // namespace qma

struct qma_layer {
  qma::Layer L;
};

namespace qma {
// Small-M kernel instances: TM = 16-token tiles per workgroup (1, 2 or 4),
// NTW = 16-column weight tiles per wave (1, 2 or 4). A workgroup has 4 waves;
// waves_k of them split K and 4 / waves_k split the columns, so
// block_n = 16 * NTW * (4 / waves_k).
// * Shared-row kernel: the four waves side by side (waves_k 1) over 2 or 4
//   column tiles each, the token rows staged once per workgroup in LDS;
//   TM * NTW <= 8 accumulator tiles per wave.
// * Per-wave-row kernel: every other shape (waves splitting K, or one
//   column tile per wave). Each wave holds its token rows in registers for
//   the whole prefetch depth, so only TM * NTW <= 4 fits the register file
//   without spilling.
constexpr bool small_m_shared_rows(int tm, int ntw, int wk) {
  return wk == 1 && (tm == 1 || tm == 2 || tm == 4) && (ntw == 2 || ntw == 4) && tm * ntw <= 8;
}
constexpr bool small_m_wave_rows(int tm, int ntw, int wk) {
  return (wk == 2 || wk == 4 || (wk == 1 && ntw == 1)) && (tm == 1 || tm == 2 || tm == 4) &&
         (ntw == 1 || ntw == 2 || ntw == 4) && tm * ntw <= 4;
}
constexpr bool small_m_supported(int tm, int ntw, int wk) {
  return small_m_shared_rows(tm, ntw, wk) || small_m_wave_rows(tm, ntw, wk);
}
// The prefetch depth (128-wide K chunks in flight per wave) of the
// per-wave-row kernel, sized to a ~160 VGPR budget.
constexpr int small_m_depth(int tm, int ntw) {
  const int per = ntw * 6 + tm * 16;
  const int fixed = ntw * tm * 4 + tm * 4 + 30;
  const int d = (160 - fixed) / per;
  return d < 2 ? 2 : (d > 4 ? 4 : d);
}
}  // namespace qma
