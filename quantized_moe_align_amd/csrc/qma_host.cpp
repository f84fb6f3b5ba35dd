// Host layer of libqma: status and error text, the quantisation-scheme
// check, layers and their profile, the planner, argument validation and
// the routing validators. Nothing here touches the GPU except the
// validators' read-back and the calls into the launchers.
//
// Passages followed (see include/qma.h for the page titles):
//   [release] runtime considerations: unsupported schemes fail at load; the
//     EP/TP profile comes from the projection shapes with no shard args;
//     the indexed kernels accept over-allocated routing buffers and are
//     graph-capturable when routing validation is off.
//   [release] indexed techniques: the tok_e block-M rule with threshold 80;
//     the stream-K gate (here split-K; a stream-K schedule that cuts items
//     in K inside a CU's share is accepted from edited plans).
//   [release] grouped techniques: BN256 only with enough N tiles (here the
//     wider of two workgroup widths); BLOCK_M from the expected token
//     count; a buffered K depth of about 512, up to about 768 for large
//     masked tiles.
//   [announce] scheduling section: the schedule follows routed tokens per
//     expert; profile and layout are fixed at load.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "qma_internal.h"

using qma::Layer;

namespace {

thread_local std::string g_detail;

qma_status fail(qma_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
qma_status fail(qma_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

qma_status ok() {
  g_detail.clear();
  return QMA_OK;
}

qma_status hip_status(int err, const char* what) {
  if (err == 0) return ok();
  return fail(QMA_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int32_t infer_profile(int32_t E, int32_t N, int32_t K) {
  (void)E;
  // gate_up maps hidden -> 2*I (K >= N in every MoE share seen); down maps
  // I -> hidden. A tensor-parallel share cuts I by the TP degree, so its
  // hidden / I ratio is large; an expert-parallel share keeps I whole.
  const bool gate_up = K >= N;
  const int64_t I = gate_up ? N / 2 : K;
  const int64_t H = gate_up ? K : N;
  if (I <= 0) return QMA_PROFILE_GENERIC;
  const bool tp = H >= 8 * I;
  if (gate_up) return tp ? QMA_PROFILE_TP_GATE_UP : QMA_PROFILE_EP_GATE_UP;
  return tp ? QMA_PROFILE_TP_DOWN : QMA_PROFILE_EP_DOWN;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

void plan_small_m(const Layer& L, int32_t bm, int32_t tiles_m, qma_plan_t* p) {
  p->kernel = QMA_KERNEL_SMALL_M;
  p->block_m = bm;
  const int tm = bm / 16;
  int wk, ntw = 0;
  if (tm <= 2) {
    // 16- and 32-row tiles: one K partition, the four waves side by side,
    // token rows shared through LDS (16 * 4 * ntw columns per workgroup).
    // 16-row tiles take 128 columns, except with short K where the
    // workgroup streams column blocks (below) and the wider block is better.
    wk = 1;
    ntw = (tm == 2 || L.k_chunks < qma::kStreamChunks) ? 4 : 2;
    while (ntw > 1 && L.N % (64 * ntw) != 0) ntw /= 2;
    // Wave-aware width: the narrower width when the wide one leaves CUs
    // without a workgroup, down to 128 columns; an underfilled grid is then
    // left to split-K, or below (64 columns) when K is too short to split.
    if (ntw > 2 && (int64_t)tiles_m * (L.N / (64 * ntw)) < qma::kNumCUs &&
        L.N % (64 * (ntw / 2)) == 0)
      ntw /= 2;
    // 16-row tiles with long K and wide N (>= 8 blocks of 256) take 256
    // columns when that still fills a whole round of three workgroups per CU
    // (the EP8 gate_up share: 48 tiles x 16 blocks = 768 workgroups;
    // measured 134.4 vs 136.9 us against 128 columns). With fewer tiles (the
    // EP16 share: 384 workgroups) the wide block leaves half the slots empty
    // and was 27 % slower; on the narrow TP8 gate_up share (N = 512, 2
    // blocks per tile) it was 1 % slower.
    if (tm == 1 && ntw == 2 && L.k_chunks >= 4 * qma::kStreamChunks && L.N % 256 == 0 &&
        L.N / 256 >= 8 && (int64_t)tiles_m * (L.N / 256) >= 3 * qma::kNumCUs)
      ntw = 4;
  } else {
    // 64-row tiles: the shared-row kernel at 128 columns (four waves side by
    // side, two column tiles each), its rows staged once per workgroup; an
    // underfilled grid is left to split-K as above.
    wk = 1;
    ntw = 2;
  }
  if (L.N % (16 * (4 / wk) * ntw) != 0) {
    // odd widths (N a multiple of 16 only): one tile per wave, waves on K
    wk = 4;
    ntw = 1;
  }
  const int wn = 4 / wk;
  p->waves_k = wk;
  p->block_n = 16 * wn * ntw;
  const int32_t tiles =
      (int32_t)std::min<int64_t>((int64_t)tiles_m * (L.N / p->block_n), 1 << 30);
  p->est_tiles = tiles;
  // Split-K gate: only when the grid holds fewer than two workgroups per
  // CU. It then aims at three per CU (one round of the gang schedule),
  // never below kSplitChunks 128-wide K chunks per split.
  // * An EP32 gate_up share, 384 tiles: split 2 on the shared-row kernel
  //   ran 42.1 us, 41.2 us as a gang, against 48.0 us for two wave pairs
  //   splitting K inside the workgroup, the earlier rule for one to two
  //   workgroups per CU; before the tiles were folded over the XCDs that
  //   order was reversed.
  // * EP128 gate_up, 96 tiles, K = 56 chunks: split 2/3/4/6/8 ran
  //   29.9/25.6/23.0/22.5/22.0 us with the tiles folded over all XCDs, and
  //   unsplit 45 us; down, 168 tiles, K = 16 chunks: split 2 was no faster
  //   than unsplit.
  int32_t split = 1;
  if (tiles < 2 * qma::kNumCUs) {
    const int32_t max_split = std::max<int32_t>(1, (int32_t)(L.k_chunks / qma::kSplitChunks));
    split = std::min<int32_t>(
        {ceil_div(qma::kGangGroups * qma::kNumCUs, std::max(tiles, 1)), max_split, 8});
    split = std::max<int32_t>(split, 1);
  }
  // An underfilled grid that K is too short to split (an EP128 down share:
  // 3 tiles x 56 blocks of 128 columns, 16 chunks) takes 64-column blocks,
  // the four waves splitting K over all four 16-column tiles, for twice the
  // workgroups: 16.7 -> 13.2 us. (With long K, split-K stays ahead: EP128
  // gate_up at 64 columns and split 2 ran 21.6 us against 23.0 at 128 and
  // split 4.)
  if (split == 1 && tiles < qma::kNumCUs && tm == 1 && wk == 1 && L.N % 64 == 0 &&
      L.k_chunks >= qma::kStreamChunks) {
    wk = 4;
    ntw = 4;                 // one wave column of four 16-column tiles
    p->waves_k = wk;
    p->block_n = 64;
    p->est_tiles = (int32_t)std::min<int64_t>((int64_t)tiles_m * (L.N / 64), 1 << 30);
  }
  p->split_k = split;
  // the shared-row kernel keeps two chunks in flight per wave (its LDS ring
  // and register stages); the per-wave-row kernel sizes its depth to its
  // register budget
  const int depth = qma::small_m_shared_rows(tm, ntw, wk) ? 2 : qma::small_m_depth(tm, ntw);
  p->k_depth = depth * qma::kChunkK;
  // Short K (a down projection of a narrow TP share): a workgroup that saw
  // only one or two chunks would spend its life on start-up and one memory
  // round trip. It streams several N blocks of its expert through the same
  // load pipeline instead, as long as the grid keeps >= 4 workgroups per CU.
  p->n_stream = 1;
  if (wk == 1 && split == 1 && tm == 1 && ntw >= 2 && L.k_chunks < qma::kStreamChunks) {
    const int32_t nblocks = L.N / p->block_n;
    int32_t ns =
        std::min<int32_t>(ceil_div(qma::kStreamTargetChunks, (int32_t)L.k_chunks), nblocks);
    while (ns > 1 && (int64_t)tiles_m * ceil_div(nblocks, ns) < 4 * qma::kNumCUs) --ns;
    p->n_stream = std::max<int32_t>(ns, 1);
  }
  // Gang schedule: where the items of a shared-row plan fill one round of
  // kGangGroups lock-step groups on every CU (5/6 of the slots or more),
  // at this width or the other one, each CU runs one workgroup holding all
  // of its items. As separate workgroups they end staggered: on the EP8
  // decode gate_up share the three on a CU ran 84, 104 and 120 us, and the
  // CU streamed at 57 % of its full rate once one was left. Measured, same
  // box: EP8 decode gate_up 127-129 -> 119-121 us, TP8 gate_up (256
  // columns) 129-130 -> 121-122 us, masked gate_up 157 -> 149-152 us.
  p->schedule = QMA_SCHEDULE_SEMI_STATIC;
  if (wk == 1 && p->n_stream == 1 && L.k_chunks >= qma::kStreamChunks) {
    const int64_t slots = (int64_t)qma::kGangGroups * qma::kNumCUs;
    // a split plan keeps its width (its split was sized for it)
    const int cands[3] = {ntw, split > 1 ? ntw : 4, split > 1 ? ntw : 2};
    for (const int cand : cands) {
      if (!qma::small_m_shared_rows(tm, cand, 1) || L.N % (64 * cand) != 0) continue;
      // token tiles (folded into column-block groups where few) are dealt
      // to the 8 XCDs in turn: the fullest XCD must fit one round too (an
      // EP32 down share without folding, 12 tiles x 56 blocks, had 112 items
      // on four XCDs and ran 40.9 us this way against 28.6 us semi-static)
      const int64_t nbc = L.N / (64 * cand);
      const int64_t items = (int64_t)tiles_m * nbc * split;
      const int f = qma::xcd_fold(tiles_m, nbc);
      const int64_t per_xcd = ceil_div((int64_t)tiles_m * f, 8) * (nbc / f) * split;
      if (per_xcd > slots / 8 || 6 * items < qma::kGangMinFill * slots) continue;
      p->block_n = 64 * cand;
      p->est_tiles = (int32_t)(items / split);
      p->schedule = QMA_SCHEDULE_GANG;
      break;
    }
  }
}

// Large-M kernel: 128-token tiles, 256 columns per workgroup.
bool large_m_fits(const Layer& L) { return L.N % 256 == 0; }

void plan_large_m(const Layer& L, int32_t bm, int32_t tiles_m, qma_plan_t* p) {
  p->kernel = QMA_KERNEL_LARGE_M;
  p->block_m = bm;
  p->block_n = 256;
  p->waves_k = 1;
  p->k_depth = 2 * qma::kChunkK;
  const int32_t tiles = (int32_t)std::min<int64_t>((int64_t)tiles_m * (L.N / 256), 1 << 30);
  p->est_tiles = tiles;
  int32_t split = 1;
  if (tiles < qma::kNumCUs) {
    const int32_t max_split = std::max<int32_t>(1, (int32_t)(L.k_chunks / 4));
    split = std::min<int32_t>({ceil_div(qma::kNumCUs, std::max(tiles, 1)), max_split, 8});
    split = std::max<int32_t>(split, 1);
  }
  p->split_k = split;
}

void plan_common(const Layer& L, qma_plan_t* p) {
  std::memset(p, 0, sizeof(*p));
  p->path = L.path;
  p->num_experts = L.E;
  p->n = L.N;
  p->k = L.K;
  p->profile = L.profile;
  p->split_k = 1;
  p->n_stream = 1;
}

// Activations are addressed with 32-bit buffer offsets.
qma_status check_a_bytes(int64_t rows, int32_t K) {
  if (rows * K * 2 >= (1ll << 31))
    return fail(QMA_ERR_INVALID_ARG, "activation of %lld x %d bf16 exceeds 2 GiB; split the call",
                (long long)rows, K);
  return ok();
}

// The semi-static grid covers every (tile, column block, split) the host
// can bound: the tile count padded to the 8 XCDs, times the column blocks
// one workgroup does not stream, times the splits. Workgroup indices must
// stay below 2^24.
qma_status check_grid(int64_t num_tiles, const qma_plan_t* plan) {
  const int64_t tiles_pad = (num_tiles + 7) / 8 * 8;
  const int64_t nblocks = plan->n / plan->block_n;
  const int64_t per = (nblocks + plan->n_stream - 1) / plan->n_stream;
  if (tiles_pad * per * plan->split_k >= (1ll << 24))
    return fail(QMA_ERR_INVALID_ARG, "%lld tiles x %lld column blocks x %d splits exceed "
                "2^24 workgroups; split the call", (long long)num_tiles, (long long)per,
                plan->split_k);
  return ok();
}

qma_status check_layer_plan(const qma_layer_t* layer, const qma_plan_t* plan,
                            int32_t path) {
  if (!layer || !plan) return fail(QMA_ERR_INVALID_ARG, "null layer or plan");
  const Layer& L = layer->L;
  if (L.path != path)
    return fail(QMA_ERR_INVALID_ARG, "layer path %d does not match call (%d)",
                L.path, path);
  if (plan->path != L.path || plan->n != L.N || plan->k != L.K ||
      plan->num_experts != L.E)
    return fail(QMA_ERR_INVALID_ARG, "plan was made for another layer");
  if (plan->kernel != QMA_KERNEL_SMALL_M && plan->kernel != QMA_KERNEL_LARGE_M &&
      plan->kernel != QMA_KERNEL_LARGE_M_PC)
    return fail(QMA_ERR_INVALID_ARG, "plan has unknown kernel %d", plan->kernel);
  const bool large = plan->kernel != QMA_KERNEL_SMALL_M;
  if (large && (plan->block_m != 128 || plan->block_n != 256 || L.N % 256 != 0))
    return fail(QMA_ERR_INVALID_ARG, "large-M plan needs block 128 x 256 and N %% 256 == 0");
  if (plan->kernel == QMA_KERNEL_LARGE_M_PC && plan->split_k != 1)
    return fail(QMA_ERR_INVALID_ARG, "the producer/consumer large-M kernel takes no split-K");
  if (plan->block_m < 16 || plan->block_m % 16 != 0 ||
      (plan->kernel == QMA_KERNEL_SMALL_M && plan->block_m > 64))
    return fail(QMA_ERR_INVALID_ARG, "plan has bad block_m %d", plan->block_m);
  if (plan->split_k < 1 || plan->split_k > 8)
    return fail(QMA_ERR_INVALID_ARG, "plan has bad split_k %d", plan->split_k);
  // every K partition must own at least one 128-wide chunk
  if (plan->split_k > L.k_chunks)
    return fail(QMA_ERR_INVALID_ARG, "split_k %d exceeds the %lld K chunks of 128", plan->split_k,
                (long long)L.k_chunks);
  const bool gang_ok =
      plan->kernel == QMA_KERNEL_SMALL_M && plan->waves_k == 1 && plan->n_stream == 1 &&
      (plan->block_n == 128 || plan->block_n == 256) && plan->block_m % 16 == 0 &&
      qma::small_m_shared_rows(plan->block_m / 16, plan->block_n / 64, 1);
  const bool stream_k_ok = gang_ok && L.path == QMA_PATH_INDEXED && plan->split_k == 1 &&
                           plan->block_m <= 32 && L.k_chunks >= qma::kStreamChunks;
  if (plan->schedule != QMA_SCHEDULE_SEMI_STATIC &&
      !(plan->schedule == QMA_SCHEDULE_GANG && gang_ok) &&
      !(plan->schedule == QMA_SCHEDULE_STREAM_K && stream_k_ok) &&
      (plan->schedule != QMA_SCHEDULE_DYNAMIC || plan->kernel != QMA_KERNEL_SMALL_M ||
       plan->waves_k != 1 || plan->split_k != 1 || plan->n_stream != 1 ||
       (plan->block_m != 16 && plan->block_m != 32) ||
       (plan->block_n != 128 && plan->block_n != 256)))
    return fail(QMA_ERR_INVALID_ARG, "plan has bad schedule %d", plan->schedule);
  if (plan->n_stream < 1 || plan->n_stream > 64 ||
      (plan->n_stream > 1 && (plan->kernel != QMA_KERNEL_SMALL_M || plan->waves_k != 1 ||
                              plan->split_k != 1 || plan->block_m != 16 ||
                              (plan->block_n != 128 && plan->block_n != 256))))
    return fail(QMA_ERR_INVALID_ARG, "plan has bad n_stream %d", plan->n_stream);
  if (plan->block_n != 16 && plan->block_n != 32 && plan->block_n != 64 &&
      plan->block_n != 128 && plan->block_n != 256)
    return fail(QMA_ERR_INVALID_ARG, "plan has bad block_n %d", plan->block_n);
  if (L.N % plan->block_n != 0)
    return fail(QMA_ERR_INVALID_ARG, "block_n %d does not divide N %d",
                plan->block_n, L.N);
  if (plan->kernel == QMA_KERNEL_SMALL_M) {
    // the small-M kernel instances: 16-column tiles per wave (ntw) times the
    // waves side by side (4 / waves_k)
    const int wk = plan->waves_k;
    const int wn = (wk == 1 || wk == 2 || wk == 4) ? 4 / wk : 0;
    if (!wn || plan->block_n % (16 * wn) != 0 ||
        !qma::small_m_supported(plan->block_m / 16, plan->block_n / (16 * wn), wk))
      return fail(QMA_ERR_INVALID_ARG, "no small-M kernel for a %d x %d block with waves_k %d",
                  plan->block_m, plan->block_n, wk);
    // fused activation: each wave must hold gate and up tiles in pairs
    if (L.act && (plan->block_n / (16 * wn)) % 2 != 0)
      return fail(QMA_ERR_INVALID_ARG,
                  "a fused gate_up layer needs an even tile count per wave (block_n %d, waves_k %d)",
                  plan->block_n, wk);
  }
  if (L.act && plan->kernel == QMA_KERNEL_LARGE_M_PC)
    return fail(QMA_ERR_INVALID_ARG, "the producer/consumer kernel has no fused activation");
  return ok();
}

size_t ws_bytes_for(const qma_plan_t* p, int64_t rows) {
  size_t b = 0;
  if (p->split_k > 1) b = (size_t)p->split_k * (size_t)rows * (size_t)p->n * sizeof(float);
  if (p->schedule == QMA_SCHEDULE_DYNAMIC) b = (b + 255) / 256 * 256 + qma::kWorkCounterBytes;
  return b;
}

qma_status check_ws(const qma_plan_t* plan, int64_t rows, const void* ws,
                    size_t ws_bytes) {
  const size_t need = ws_bytes_for(plan, rows);
  if (need == 0) return ok();
  if (!ws || ws_bytes < need)
    return fail(QMA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                need, ws ? ws_bytes : (size_t)0);
  if (!aligned(ws, 16)) return fail(QMA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  return ok();
}

}  // namespace

extern "C" {

const char* qma_status_str(qma_status s) {
  switch (s) {
    case QMA_OK: return "QMA_OK";
    case QMA_ERR_INVALID_ARG: return "QMA_ERR_INVALID_ARG";
    case QMA_ERR_UNSUPPORTED: return "QMA_ERR_UNSUPPORTED";
    case QMA_ERR_ROUTING: return "QMA_ERR_ROUTING";
    case QMA_ERR_WORKSPACE: return "QMA_ERR_WORKSPACE";
    case QMA_ERR_HIP: return "QMA_ERR_HIP";
  }
  return "QMA_ERR_UNKNOWN";
}

const char* qma_last_error_detail(void) { return g_detail.c_str(); }

const char* qma_version(void) { return "qma 0.1 gfx950"; }

qma_status qma_layer_create(const qma_quant_desc* q, int32_t E, int32_t N,
                            int32_t K, qma_path path, qma_layer_t** out) {
  return qma_layer_create_ex(q, E, N, K, path, 0, out);
}

qma_status qma_layer_create_ex(const qma_quant_desc* q, int32_t E, int32_t N, int32_t K,
                               qma_path path, uint32_t flags, qma_layer_t** out) {
  if (!q || !out) return fail(QMA_ERR_INVALID_ARG, "null descriptor or out");
  *out = nullptr;
  if (q->weight_bits != 4)
    return fail(QMA_ERR_UNSUPPORTED, "weight_bits %d: only uint4 is supported", q->weight_bits);
  if (q->zero_point != 8)
    return fail(QMA_ERR_UNSUPPORTED, "zero_point %d: only 8 is supported", q->zero_point);
  if (q->group_size != 32)
    return fail(QMA_ERR_UNSUPPORTED, "group_size %d: only 32 is supported", q->group_size);
  if (q->scale_dtype != QMA_DTYPE_BF16)
    return fail(QMA_ERR_UNSUPPORTED, "scale dtype %d: only bf16 scales are supported", q->scale_dtype);
  if (q->act_dtype != QMA_DTYPE_BF16)
    return fail(QMA_ERR_UNSUPPORTED, "activation dtype %d: only bf16 is supported", q->act_dtype);
  if (q->pack_format != QMA_PACK_INT32_K8)
    return fail(QMA_ERR_UNSUPPORTED, "pack format %d: only int32 K8 is supported", q->pack_format);
  if (path != QMA_PATH_INDEXED && path != QMA_PATH_GROUPED_CONTIGUOUS &&
      path != QMA_PATH_GROUPED_MASKED)
    return fail(QMA_ERR_INVALID_ARG, "unknown path %d", (int)path);
  if (E < 1 || N < 16 || K < 128)
    return fail(QMA_ERR_INVALID_ARG, "bad shape E=%d N=%d K=%d", E, N, K);
  if (N % 16 != 0) return fail(QMA_ERR_INVALID_ARG, "N=%d is not a multiple of 16", N);
  if (K % 128 != 0) return fail(QMA_ERR_INVALID_ARG, "K=%d is not a multiple of 128", K);
  if (flags & ~(uint32_t)QMA_LAYER_FUSE_SILU_MUL)
    return fail(QMA_ERR_INVALID_ARG, "unknown layer flags 0x%x", flags);
  const bool fuse = flags & QMA_LAYER_FUSE_SILU_MUL;
  if (fuse && N % 64 != 0)
    return fail(QMA_ERR_INVALID_ARG, "a fused gate_up layer needs N %% 64 == 0 (N=%d)", N);
  auto* l = new (std::nothrow) qma_layer_t;
  if (!l) return fail(QMA_ERR_INVALID_ARG, "out of host memory");
  Layer& L = l->L;
  L.E = E;
  L.N = N;
  L.K = K;
  L.path = path;
  L.act = fuse ? 1 : 0;
  L.profile = infer_profile(E, N, K);
  L.n_tiles = N / qma::kTileN;
  L.k_chunks = K / qma::kChunkK;
  // one expert's packed weights are addressed with 32-bit offsets
  if ((int64_t)L.n_tiles * L.k_chunks * qma::kWBlockBytes >= (1ll << 31)) {
    delete l;
    return fail(QMA_ERR_INVALID_ARG, "N=%d x K=%d: one expert's packed weights exceed 2 GiB", N, K);
  }
  L.wg_log2 = ((L.profile == QMA_PROFILE_EP_GATE_UP || L.profile == QMA_PROFILE_TP_GATE_UP) &&
               L.n_tiles % (1 << qma::kGateUpGroupLog2) == 0)
                  ? qma::kGateUpGroupLog2
                  : 0;
  L.w_bytes = (size_t)E * L.n_tiles * L.k_chunks * qma::kWBlockBytes;
  L.s_bytes = (size_t)E * L.n_tiles * L.k_chunks * qma::kSBlockBytes;
  *out = l;
  return ok();
}

void qma_layer_destroy(qma_layer_t* layer) { delete layer; }

qma_status qma_layer_info(const qma_layer_t* layer, int32_t* E, int32_t* N,
                          int32_t* K, int32_t* path, int32_t* profile) {
  if (!layer) return fail(QMA_ERR_INVALID_ARG, "null layer");
  if (E) *E = layer->L.E;
  if (N) *N = layer->L.N;
  if (K) *K = layer->L.K;
  if (path) *path = layer->L.path;
  if (profile) *profile = layer->L.profile;
  return ok();
}

size_t qma_packed_weight_bytes(const qma_layer_t* layer) {
  if (!layer) return 0;
  return layer->L.w_bytes + layer->L.s_bytes;
}

qma_status qma_prepack(const qma_layer_t* layer, const int32_t* qweight,
                       const uint16_t* scales, void* packed, void* stream) {
  if (!layer || !qweight || !scales || !packed)
    return fail(QMA_ERR_INVALID_ARG, "null argument");
  if (!aligned(packed, 256)) return fail(QMA_ERR_INVALID_ARG, "packed buffer not 256-byte aligned");
  if (!aligned(qweight, 4) || !aligned(scales, 2))
    return fail(QMA_ERR_INVALID_ARG, "misaligned qweight or scales");
  return hip_status(qma::launch_prepack(layer->L, qweight, scales, packed, stream),
                    "prepack launch");
}

qma_status qma_plan_indexed(const qma_layer_t* layer, int32_t T, int32_t topk,
                            int32_t force_block_m, qma_plan_t* out) {
  if (!layer || !out) return fail(QMA_ERR_INVALID_ARG, "null layer or out");
  const Layer& L = layer->L;
  if (L.path != QMA_PATH_INDEXED) return fail(QMA_ERR_INVALID_ARG, "layer is not INDEXED");
  if (T < 0 || topk < 1) return fail(QMA_ERR_INVALID_ARG, "bad T=%d topk=%d", T, topk);
  const int64_t R = (int64_t)T * topk;
  if (R >= (1ll << 30)) return fail(QMA_ERR_INVALID_ARG, "T*topk too large");
  plan_common(L, out);
  out->rows = (int32_t)R;
  const double tok_e = (double)R / L.E;
  out->tok_e_x100 = (int32_t)std::lround(tok_e * 100.0);
  const int64_t e_active = std::min<int64_t>(L.E, std::max<int64_t>(R, 1));
  if (force_block_m != 0 && force_block_m != 16 && force_block_m != 32 &&
      force_block_m != 64 && force_block_m != 128)
    return fail(QMA_ERR_INVALID_ARG, "force_block_m %d not in {16,32,64,128}", force_block_m);
  if (force_block_m == 128 && !large_m_fits(L))
    return fail(QMA_ERR_INVALID_ARG, "block_m %d needs N %% 256 == 0 (N=%d)", force_block_m, L.N);
  // At or above 80 routed rows per expert the large-M kernel amortises the
  // dequantisation over 128 tokens; below, the small-M kernel takes the
  // smallest of 16, 32, 64 rows that covers tok_e.
  const bool large = force_block_m == 128 ||
                     (force_block_m == 0 && tok_e >= 80.0 && large_m_fits(L));
  if (large) {
    const int64_t per_e = std::max<int64_t>(1, ceil_div((int64_t)std::ceil(tok_e), 128));
    plan_large_m(L, 128, (int32_t)std::min<int64_t>(e_active * per_e, 1 << 30), out);
    return ok();
  }
  const int32_t bm = force_block_m != 0 ? force_block_m
                                        : (tok_e <= 16 ? 16 : (tok_e <= 32 ? 32 : 64));
  const int64_t per_e = std::max<int64_t>(1, ceil_div((int64_t)std::ceil(tok_e), bm));
  plan_small_m(L, bm, (int32_t)std::min<int64_t>(e_active * per_e, 1 << 30), out);
  return ok();
}

qma_status qma_plan_grouped(const qma_layer_t* layer, int32_t m_rows_or_budget,
                            int32_t expected_m, qma_plan_t* out) {
  if (!layer || !out) return fail(QMA_ERR_INVALID_ARG, "null layer or out");
  const Layer& L = layer->L;
  plan_common(L, out);
  if (L.path == QMA_PATH_GROUPED_CONTIGUOUS) {
    const int32_t M = m_rows_or_budget;
    if (M < 0 || M % 128 != 0)
      return fail(QMA_ERR_INVALID_ARG, "contiguous M=%d is not a multiple of 128", M);
    out->rows = M;
    const double tok_e = (double)M / L.E;
    out->tok_e_x100 = (int32_t)std::lround(tok_e * 100.0);
    // Every expert's rows come padded to a multiple of 128, so each 128-row
    // tile holds one expert and the large-M kernel applies whenever N allows,
    // however many experts are empty (M/E says nothing about that).
    if (large_m_fits(L))
      plan_large_m(L, 128, std::max(1, M / 128), out);
    else
      plan_small_m(L, 64, std::max(1, M / 64), out);
    return ok();
  }
  if (L.path == QMA_PATH_GROUPED_MASKED) {
    const int32_t Mb = m_rows_or_budget;
    if (Mb < 1 || expected_m < 0 || expected_m > Mb)
      return fail(QMA_ERR_INVALID_ARG, "bad budget %d / expected_m %d", Mb, expected_m);
    if ((int64_t)Mb * L.E >= (1ll << 30)) return fail(QMA_ERR_INVALID_ARG, "E*budget too large");
    out->rows = Mb * L.E;
    out->tok_e_x100 = expected_m * 100;
    const int32_t bm = expected_m <= 16 ? 16 : (expected_m <= 32 ? 32 : 64);
    plan_small_m(L, bm, L.E * std::max(1, ceil_div(std::max(expected_m, 1), bm)), out);
    out->expected_m = expected_m;
    return ok();
  }
  return fail(QMA_ERR_INVALID_ARG, "layer is not a grouped layer");
}

size_t qma_workspace_bytes(const qma_plan_t* plan) {
  if (!plan) return 0;
  return ws_bytes_for(plan, plan->rows);
}

qma_status qma_align_sizes(int32_t T, int32_t topk, int32_t E, int32_t block_m,
                           int32_t* sorted_cap, int32_t* blocks_cap) {
  if (T < 0 || topk < 1 || E < 1 || block_m < 1)
    return fail(QMA_ERR_INVALID_ARG, "bad T=%d topk=%d E=%d block_m=%d", T, topk, E, block_m);
  const int64_t cap = (int64_t)T * topk + (int64_t)E * (block_m - 1);
  if (cap >= (1ll << 31) - block_m) return fail(QMA_ERR_INVALID_ARG, "capacity overflows int32");
  if (sorted_cap) *sorted_cap = (int32_t)cap;
  if (blocks_cap) *blocks_cap = (int32_t)((cap + block_m - 1) / block_m);
  return ok();
}

qma_status qma_moe_align(const int32_t* topk_ids, int32_t T, int32_t topk,
                         int32_t E, int32_t block_m, int32_t* sorted_ids,
                         int32_t* expert_ids, int32_t* num_tokens_padded,
                         int32_t sorted_cap, void* stream) {
  int32_t need = 0;
  qma_status s = qma_align_sizes(T, topk, E, block_m, &need, nullptr);
  if (s != QMA_OK) return s;
  if (E > qma::kMaxExperts) return fail(QMA_ERR_INVALID_ARG, "E=%d exceeds %d", E, qma::kMaxExperts);
  if (sorted_cap < need)
    return fail(QMA_ERR_INVALID_ARG, "sorted_cap %d below the bound %d", sorted_cap, need);
  if ((T > 0 && !topk_ids) || !sorted_ids || !expert_ids || !num_tokens_padded)
    return fail(QMA_ERR_INVALID_ARG, "null buffer");
  return hip_status(qma::launch_moe_align(topk_ids, T * topk, E, block_m, sorted_ids,
                                          expert_ids, num_tokens_padded, sorted_cap,
                                          stream),
                    "moe_align launch");
}

}  // extern "C"

namespace {

template <typename T>
qma_status read_back(std::vector<T>& dst, const T* src, size_t n, hipStream_t st) {
  dst.resize(n);
  if (n == 0) return ok();
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return hip_status((int)e, "validation read-back");
}

}  // namespace

extern "C" {

qma_status qma_validate_routing(const int32_t* topk_ids, int32_t T, int32_t topk,
                                int32_t E, int32_t block_m,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_tokens_padded, int32_t sorted_cap,
                                void* stream) {
  if (T < 0 || topk < 1 || E < 1 || block_m < 1 || sorted_cap < 0)
    return fail(QMA_ERR_INVALID_ARG, "bad sizes");
  if ((T > 0 && !topk_ids) || !sorted_ids || !expert_ids || !num_tokens_padded)
    return fail(QMA_ERR_INVALID_ARG, "null buffer");
  hipStream_t st = (hipStream_t)stream;
  const int64_t R = (int64_t)T * topk;
  const int64_t blocks = (sorted_cap + block_m - 1) / block_m;
  std::vector<int32_t> ids, sorted, experts, ntp;
  qma_status s;
  if ((s = read_back(ids, topk_ids, (size_t)R, st)) != QMA_OK) return s;
  if ((s = read_back(sorted, sorted_ids, (size_t)sorted_cap, st)) != QMA_OK) return s;
  if ((s = read_back(experts, expert_ids, (size_t)blocks, st)) != QMA_OK) return s;
  if ((s = read_back(ntp, num_tokens_padded, 1, st)) != QMA_OK) return s;
  for (int64_t i = 0; i < R; ++i)
    if (ids[i] < -1 || ids[i] >= E)
      return fail(QMA_ERR_ROUTING, "topk_ids[%lld] = %d outside [-1, %d)", (long long)i, ids[i], E);
  // The buffers moe_align defines for these ids, recomputed on the host: a
  // stable counting sort of the slots by expert, each expert padded with the
  // sentinel R to a multiple of block_m, then the tails.
  std::vector<int64_t> count((size_t)E, 0), start((size_t)E + 1, 0);
  for (int64_t i = 0; i < R; ++i)
    if (ids[i] >= 0) ++count[(size_t)ids[i]];
  for (int32_t e = 0; e < E; ++e)
    start[(size_t)e + 1] = start[(size_t)e] + (count[(size_t)e] + block_m - 1) / block_m * block_m;
  const int64_t want_ntp = start[(size_t)E];
  if (want_ntp > sorted_cap)
    return fail(QMA_ERR_ROUTING, "sorted_cap %d is below the padded length %lld", sorted_cap,
                (long long)want_ntp);
  if (ntp[0] != want_ntp)
    return fail(QMA_ERR_ROUTING, "num_tokens_padded %d, expected %lld", ntp[0],
                (long long)want_ntp);
  std::vector<int32_t> want_sorted((size_t)sorted_cap, (int32_t)R);
  std::vector<int64_t> next(start.begin(), start.end() - 1);
  for (int64_t i = 0; i < R; ++i)
    if (ids[i] >= 0) want_sorted[(size_t)next[(size_t)ids[i]]++] = (int32_t)i;
  std::vector<int32_t> want_experts((size_t)blocks, -1);
  for (int32_t e = 0; e < E; ++e)
    for (int64_t b = start[(size_t)e] / block_m; b < start[(size_t)e + 1] / block_m; ++b)
      want_experts[(size_t)b] = e;
  for (int64_t p = 0; p < sorted_cap; ++p) {
    if (sorted[(size_t)p] == want_sorted[(size_t)p]) continue;
    const char* where = p >= want_ntp ? "tail past num_tokens_padded"
                        : want_sorted[(size_t)p] == R ? "expert padding"
                                                      : "an expert's slot list";
    return fail(QMA_ERR_ROUTING, "sorted_ids[%lld] = %d, expected %d (%s)", (long long)p,
                sorted[(size_t)p], want_sorted[(size_t)p], where);
  }
  for (int64_t b = 0; b < blocks; ++b) {
    if (experts[(size_t)b] == want_experts[(size_t)b]) continue;
    return fail(QMA_ERR_ROUTING, "expert_ids[%lld] = %d, expected %d (%s)", (long long)b,
                experts[(size_t)b], want_experts[(size_t)b],
                b * block_m >= want_ntp ? "tail" : "routed block");
  }
  return ok();
}

qma_status qma_validate_contiguous(const int32_t* m_indices, int32_t M, int32_t E,
                                   void* stream) {
  if (M < 0 || M % 128 != 0 || E < 1) return fail(QMA_ERR_INVALID_ARG, "bad M=%d or E=%d", M, E);
  if (M > 0 && !m_indices) return fail(QMA_ERR_INVALID_ARG, "null m_indices");
  std::vector<int32_t> m;
  qma_status s = read_back(m, m_indices, (size_t)M, (hipStream_t)stream);
  if (s != QMA_OK) return s;
  for (int32_t b = 0; b < M; b += 128) {
    const int32_t e = m[b];
    if (e < -1 || e >= E) return fail(QMA_ERR_ROUTING, "m_indices[%d] = %d outside [-1, %d)", b, e, E);
    bool pad = e < 0;
    for (int32_t r = b; r < b + 128; ++r) {
      if (m[r] == -1) { pad = true; continue; }
      if (pad || m[r] != e)
        return fail(QMA_ERR_ROUTING, "m_indices[%d] = %d breaks the one-expert 128-row block at %d",
                    r, m[r], b);
    }
  }
  return ok();
}

qma_status qma_indexed_gemm(const qma_layer_t* layer, const qma_plan_t* plan,
                            const uint16_t* a, int32_t a_rows, int32_t a_row_div,
                            const void* packed_w, const int32_t* sorted_ids,
                            const int32_t* expert_ids, const int32_t* num_tokens_padded,
                            int32_t sorted_cap, int32_t num_slots,
                            const float* topk_weights, uint16_t* c, void* ws,
                            size_t ws_bytes, void* stream) {
  qma_status s = check_layer_plan(layer, plan, QMA_PATH_INDEXED);
  if (s != QMA_OK) return s;
  if (a_rows < 0 || a_row_div < 1 || num_slots < 0 || sorted_cap < 0)
    return fail(QMA_ERR_INVALID_ARG, "bad sizes");
  if ((int64_t)a_rows * a_row_div < num_slots)
    return fail(QMA_ERR_INVALID_ARG, "a has %d rows; %d slots / %d need more", a_rows,
                num_slots, a_row_div);
  // The grid covers ceil(sorted_cap / block_m) blocks; below the moe_align
  // bound, routed blocks past it would be skipped with no error.
  const int64_t cap_bound = (int64_t)num_slots + (int64_t)layer->L.E * (plan->block_m - 1);
  if (sorted_cap < cap_bound)
    return fail(QMA_ERR_INVALID_ARG, "sorted_cap %d below the bound %lld (num_slots + E*(block_m-1))",
                sorted_cap, (long long)cap_bound);
  if (!a || !packed_w || !sorted_ids || !expert_ids || !num_tokens_padded || !c)
    return fail(QMA_ERR_INVALID_ARG, "null buffer");
  if (!aligned(a, 16) || !aligned(c, 16) || !aligned(packed_w, 256))
    return fail(QMA_ERR_INVALID_ARG, "a/c must be 16-byte and packed_w 256-byte aligned");
  if ((s = check_ws(plan, num_slots, ws, ws_bytes)) != QMA_OK) return s;
  if ((s = check_a_bytes(a_rows, layer->L.K)) != QMA_OK) return s;
  if ((s = check_grid(((int64_t)sorted_cap + plan->block_m - 1) / plan->block_m, plan)) != QMA_OK)
    return s;
  if (plan->schedule == QMA_SCHEDULE_STREAM_K &&
      !qma::stream_k_fits(((int64_t)sorted_cap + plan->block_m - 1) / plan->block_m,
                          layer->L.N / plan->block_n, layer->L.k_chunks, plan->block_n / 64))
    return fail(QMA_ERR_INVALID_ARG,
                "stream-K: sorted_cap %d gives a group items of more than two token tiles "
                "(%d column blocks per tile)", sorted_cap, layer->L.N / plan->block_n);
  if (num_slots == 0) return ok();
  qma::GemmArgs g{};
  g.layer = &layer->L;
  g.plan = plan;
  g.a = a;
  g.packed = packed_w;
  g.c = c;
  g.ws = ws;
  g.mode = 0;
  g.a_row_div = a_row_div;
  g.sorted_ids = sorted_ids;
  g.expert_ids = expert_ids;
  g.ntp = num_tokens_padded;
  g.num_tiles = (sorted_cap + plan->block_m - 1) / plan->block_m;
  g.num_slots = num_slots;
  g.topk_weights = topk_weights;
  g.rows_cap = num_slots;
  g.sorted_cap = sorted_cap;
  g.a_bytes = (int64_t)a_rows * layer->L.K * 2;
  return hip_status(qma::launch_gemm(g, stream), "indexed gemm launch");
}

qma_status qma_indexed_gemm_scratch(const qma_layer_t* layer, const qma_plan_t* plan,
                                    const uint16_t* a, int32_t a_rows, int32_t a_row_div,
                                    const void* packed_w, const int32_t* sorted_ids,
                                    const int32_t* expert_ids, const int32_t* num_tokens_padded,
                                    int32_t sorted_cap, int32_t num_slots,
                                    const float* topk_weights, uint16_t* c, void* stream) {
  qma_status s = check_layer_plan(layer, plan, QMA_PATH_INDEXED);
  if (s != QMA_OK) return s;
  if (num_slots < 0) return fail(QMA_ERR_INVALID_ARG, "bad sizes");
  const size_t need = ws_bytes_for(plan, num_slots);
  if (need > qma::kScratchBytes)
    return fail(QMA_ERR_WORKSPACE,
                "this plan needs %zu bytes of workspace; the static scratch holds %zu "
                "(call qma_indexed_gemm with a workspace instead)",
                need, qma::kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const int err = qma::scratch_device_ptr(&ws);
    if (err != 0) return hip_status(err, "static scratch address");
  }
  return qma_indexed_gemm(layer, plan, a, a_rows, a_row_div, packed_w, sorted_ids, expert_ids,
                          num_tokens_padded, sorted_cap, num_slots, topk_weights, c, ws, need,
                          stream);
}

qma_status qma_grouped_contiguous_gemm(const qma_layer_t* layer, const qma_plan_t* plan,
                                       const uint16_t* a, const int32_t* m_indices,
                                       int32_t M, const void* packed_w, uint16_t* c,
                                       void* ws, size_t ws_bytes, void* stream) {
  qma_status s = check_layer_plan(layer, plan, QMA_PATH_GROUPED_CONTIGUOUS);
  if (s != QMA_OK) return s;
  if (M < 0 || M % 128 != 0) return fail(QMA_ERR_INVALID_ARG, "M=%d not a multiple of 128", M);
  if (128 % plan->block_m != 0)
    return fail(QMA_ERR_INVALID_ARG, "block_m %d does not divide 128", plan->block_m);
  if (M > plan->rows) return fail(QMA_ERR_INVALID_ARG, "M=%d exceeds the plan's %d rows", M, plan->rows);
  if (!a || !m_indices || !packed_w || !c) return fail(QMA_ERR_INVALID_ARG, "null buffer");
  if (!aligned(a, 16) || !aligned(c, 16) || !aligned(packed_w, 256))
    return fail(QMA_ERR_INVALID_ARG, "a/c must be 16-byte and packed_w 256-byte aligned");
  if ((s = check_ws(plan, M, ws, ws_bytes)) != QMA_OK) return s;
  if ((s = check_a_bytes(M, layer->L.K)) != QMA_OK) return s;
  if ((s = check_grid(M / plan->block_m, plan)) != QMA_OK) return s;
  if (M == 0) return ok();
  qma::GemmArgs g{};
  g.layer = &layer->L;
  g.plan = plan;
  g.a = a;
  g.packed = packed_w;
  g.c = c;
  g.ws = ws;
  g.mode = 1;
  g.a_row_div = 1;
  g.m_indices = m_indices;
  g.num_tiles = M / plan->block_m;
  g.num_slots = M;
  g.rows_cap = M;
  g.a_bytes = (int64_t)M * layer->L.K * 2;
  return hip_status(qma::launch_gemm(g, stream), "contiguous gemm launch");
}

qma_status qma_grouped_masked_gemm(const qma_layer_t* layer, const qma_plan_t* plan,
                                   const uint16_t* a, const int32_t* masked_m, int32_t Mb,
                                   int32_t expected_m, const void* packed_w, uint16_t* c,
                                   void* ws, size_t ws_bytes, void* stream) {
  qma_status s = check_layer_plan(layer, plan, QMA_PATH_GROUPED_MASKED);
  if (s != QMA_OK) return s;
  if (Mb < 1 || (int64_t)Mb * layer->L.E != plan->rows)
    return fail(QMA_ERR_INVALID_ARG, "budget %d does not match the plan", Mb);
  if (expected_m != plan->expected_m)
    return fail(QMA_ERR_INVALID_ARG, "expected_m %d does not match the plan's %d", expected_m,
                plan->expected_m);
  if (!a || !masked_m || !packed_w || !c) return fail(QMA_ERR_INVALID_ARG, "null buffer");
  if (!aligned(a, 16) || !aligned(c, 16) || !aligned(packed_w, 256))
    return fail(QMA_ERR_INVALID_ARG, "a/c must be 16-byte and packed_w 256-byte aligned");
  if ((s = check_ws(plan, (int64_t)Mb * layer->L.E, ws, ws_bytes)) != QMA_OK) return s;
  if ((s = check_a_bytes((int64_t)Mb * layer->L.E, layer->L.K)) != QMA_OK) return s;
  if ((s = check_grid((int64_t)(Mb + plan->block_m - 1) / plan->block_m * layer->L.E, plan)) !=
      QMA_OK)
    return s;
  qma::GemmArgs g{};
  g.layer = &layer->L;
  g.plan = plan;
  g.a = a;
  g.packed = packed_w;
  g.c = c;
  g.ws = ws;
  g.mode = 2;
  g.a_row_div = 1;
  g.masked_m = masked_m;
  g.Mb = Mb;
  g.tiles_per_expert = (Mb + plan->block_m - 1) / plan->block_m;
  g.num_tiles = g.tiles_per_expert * layer->L.E;
  g.num_slots = Mb * layer->L.E;
  g.rows_cap = Mb * layer->L.E;
  g.a_bytes = (int64_t)Mb * layer->L.E * layer->L.K * 2;
  return hip_status(qma::launch_gemm(g, stream), "masked gemm launch");
}

qma_status qma_silu_and_mul(const uint16_t* x, uint16_t* y, int64_t R, int32_t I,
                            void* stream) {
  if (R < 0 || I < 1) return fail(QMA_ERR_INVALID_ARG, "bad R=%lld I=%d", (long long)R, I);
  if (R == 0) return ok();
  if (!x || !y) return fail(QMA_ERR_INVALID_ARG, "null buffer");
  return hip_status(qma::launch_silu_and_mul(x, y, R, I, stream), "silu_and_mul launch");
}

qma_status qma_router_topk(const float* logits, int32_t T, int32_t E, int32_t topk,
                           int32_t* topk_ids, float* topk_weights, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || topk < 1 || topk > std::min(E, 16))
    return fail(QMA_ERR_INVALID_ARG, "bad sizes T=%d E=%d topk=%d", T, E, topk);
  if (T == 0) return ok();
  if (!logits || !topk_ids) return fail(QMA_ERR_INVALID_ARG, "null buffer");
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || (topk_weights && !aligned(topk_weights, 4)))
    return fail(QMA_ERR_INVALID_ARG, "buffers must be 4-byte aligned");
  return hip_status(qma::launch_router_topk(logits, T, E, topk, topk_ids, topk_weights, stream),
                    "router launch");
}

qma_status qma_moe_combine(const uint16_t* c2, const float* w, const int32_t* topk_ids,
                           int32_t E, int32_t T, int32_t topk, int32_t N, uint16_t* out,
                           void* stream) {
  if (T < 0 || topk < 1 || N < 1 || (topk_ids && E < 1))
    return fail(QMA_ERR_INVALID_ARG, "bad sizes");
  if (T == 0) return ok();
  if (!c2 || !w || !out) return fail(QMA_ERR_INVALID_ARG, "null buffer");
  return hip_status(qma::launch_combine(c2, w, topk_ids, E, T, topk, N, out, stream),
                    "combine launch");
}

}  // extern "C"
