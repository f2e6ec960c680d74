// Chunked paged prefill attention for gfx950, on the matrix cores.
//
// A chunk of T new tokens of a sequence, appended after C cached ones
// (L = C + T), brings T queries; query t sits at position C + t and attends
// causally to positions 0 .. C + t of its sequence, reading K/V through the
// block table ("PagedAttention e continuous batching", 01 · Conceito:
// the kernel follows the block table, paragraph 3; long prefills are cut
// into slices, the scheduler paragraph).  Unlike decode, many queries share
// every K/V tile, so the products are dense contractions and run as MFMA.
//
// Work decomposition.  A workgroup of 4 waves takes one tile of query rows
// of one sequence and one KV head: 128 rows = (token, head) pairs, where the
// Gw query heads of that KV head that share the tile are packed into the
// rows (Gw = 1 for MHA: 128 tokens of one head; Gw = 4 for GQA-4: 32 tokens
// x 4 heads).  Each wave owns two groups of 16 rows; every K or V^T operand
// it reads from LDS feeds one MFMA per group.  The workgroup walks the
// sequence's keys in stages of 32 tokens (two blocks) up to its last
// query's position.
//
// Per stage.  All 256 threads stage the two K tiles into LDS as they are
// (rows padded by 16 bytes against bank conflicts) and the two V tiles
// transposed (V^T, d-major, 4-token column blocks swizzled per row against
// bank conflicts), while the previous stage is computed.  A wave
// then forms S^T = K Q^T with v_mfma_f32_16x16x32_{f16,bf16}: K from LDS is
// the A operand (lane = 16 g + n holds token n, d-chunk 8 g), Q^T from
// registers the B operand (query row n, d-chunk 8 g), and the accumulator
// leaves lane (g, n) with tokens 4 g .. 4 g + 3 of each block for query row
// n.  That is the B-operand layout of the next product, so after the online
// softmax (base 2, one state per query row held by the four lanes of the
// row) P^T goes straight into O^T += V^T P^T, with V^T from LDS as the A
// operand (slot order: the 4 tokens of the first block, then the 4 of the
// second, on both sides).  Masking: keys past the query's position or past
// the context get -inf; V rows past the context are staged as zeros, so
// stale or NaN slots never reach the output.
//
// Precision.  Products of 16-bit inputs accumulate in fp32.  The softmax
// weights must become 16-bit MFMA operands, and bf16 weights alone (8-bit
// significand) put the error of short contexts above 2e-3.  So the weights
// are rounded to fp16 (11 bits) and O^T += V^T P^T runs in fp16 for both
// pool types: a bf16 pool's V is converted to fp16 while it is staged,
// which is exact for magnitudes below 2^16 (bf16 keeps 8 significant bits,
// fp16 11; below 2^-14 fp16 steps are 2^-24 apart).  A bf16 launch that
// stages a V value of magnitude 2^16 or more records its launch number in a
// device word; a second, exact pass follows every bf16 launch and runs only
// when it finds its own number there (otherwise its workgroups exit at
// once).  The exact pass keeps V in bf16 and splits each weight into a bf16
// head and a bf16 remainder (two MFMAs, ~16 bits).  Weights round to nearest
// even, two per conversion instruction.  The normaliser sums the weights the
// products use: the fp16-rounded ones (which halves the worst error of
// short rows against summing the unrounded ones), or in the exact pass the
// fp32 ones, which head + remainder match to ~16 bits.
// A row's running maximum is raised only when a score exceeds it by more
// than 2^8 in weight, and the accumulators are rescaled only in stages where
// some row's maximum moved (a wave-wide vote); otherwise the factor is
// exactly 1.
#include <atomic>
#include <cmath>
#include <cstdlib>

#include "mfma_common.h"

namespace pkv {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfRowGroups = kPrefillTileRows / (16 * kPfWaves);  // 16-row groups per wave
constexpr int kPfThreads = kWave * kPfWaves;
constexpr int kStage = 32;  // key tokens per stage (two blocks)
constexpr float kLog2eF = 1.4426950408889634f;
// Slack of the running maximum, in base-2 units: a row's maximum is raised
// (and its accumulators rescaled) only when a score exceeds it by more than
// this, so after the first keys of a long context the rescale almost never
// runs.  Weights are then at most 2^8: exact enough as fp16 (11-bit
// significand at any magnitude) or as a bf16 head + remainder, and row sums
// of up to 2^8 times the key count stay far inside fp32.
constexpr float kRescaleSlack = 8.f;

struct PrefillParams {
  const char* q;             // [total_q][H_q][D]
  float* out;                // [total_q][H_q][D]
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* work;       // [n_work][6] (sequence, tile, stage begin, stage end, split, part)
  const int32_t* q_start;    // [num_seqs + 1]
  const int32_t* split_tab;  // [n_split][2] (first partial, parts)
  int32_t* counters;         // [n_split][hgroups] completion tickets
  float* part;               // [n_partials][hgroups][tile rows] records of rec_floats
  int32_t rec_floats;        // o[D], m, l padded to whole 128-byte lines
  int32_t n_split;
  int32_t n_partials;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;             // H_q / H_kv
  int32_t hgroups_per_kv;    // group / Gw
  int32_t table_stride;
  int32_t num_blocks;
  float scale_log2;
  uint64_t overflow_launch;  // bf16 fast pass: this launch's number, recorded on overflow
  uint64_t gate_launch;      // bf16 exact pass: run only if the device word reached it
};

// Largest launch number whose fast bf16 pass staged a V value that fp16
// cannot hold (magnitude >= 2^16).  One word per device, raised with an
// atomic maximum and never lowered: launch numbers only grow, so a pass
// never misses its own record (concurrent launches can only cause an exact
// pass that was not needed).
__device__ unsigned long long g_v_overflow_launch = 0;

// 16-byte store / load at device scope: cache policy sc1, the coherence
// level the compiler gives relaxed agent-scope atomics (which it emits as
// 4-byte sc1 accesses), so records written this way are read by a
// workgroup on any XCD with no cache maintenance, in a quarter of the
// transactions.
constexpr int kCachePolicyDevice = 16;  // sc1
__device__ __forceinline__ void store_device(__amdgpu_buffer_rsrc_t r, int offset, const f4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, offset, 0, kCachePolicyDevice);
}
__device__ __forceinline__ f4 load_device(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, kCachePolicyDevice));
}

// Three waves per SIMD: the compiler then keeps the accumulators in the
// arch registers (no spills) and a CU runs three workgroups, whose MFMA and
// softmax phases overlap.
// SPLIT: the plan splits some tiles' keys into parts; without it the kernel
// carries no code for partial records (the main loop then keeps its
// registers: that code alone cost 13% on unsplit launches).
// EXACT (bf16 only): the exact pass, V staged as bf16 and the weights as a
// bf16 head + remainder; otherwise V and the weights are fp16.
template <int DT, int D, int GW, bool SPLIT, bool EXACT>
__global__ __launch_bounds__(kPfThreads, 3) void paged_prefill_kernel(const PrefillParams p) {
  constexpr bool VCONV = DT == PKV_BF16 && !EXACT;  // bf16 V staged as fp16
  constexpr bool PSPLIT = DT == PKV_BF16 && EXACT;  // weights as head + remainder
  constexpr int PVT = PSPLIT ? PKV_BF16 : PKV_F16;  // operand type of O^T += V^T P^T
  if constexpr (EXACT) {
    // one read, shared through LDS: a concurrent launch may raise the word
    // meanwhile, and the whole workgroup must take the same branch
    __shared__ int sm_run;
    if (threadIdx.x == 0)
      sm_run = __hip_atomic_load(&g_v_overflow_launch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= p.gate_launch;
    __syncthreads();
    if (!sm_run) return;
  }
  constexpr int RG = kPfRowGroups;         // 16-row groups per wave
  constexpr int TPW = 16 * RG / GW;        // query tokens per wave
  constexpr int TQ = kPfWaves * TPW;       // query tokens per workgroup
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int ROWB = D * 2;              // bytes per token row of one head
  constexpr int TILE = kBlockTokens * ROWB;
  constexpr int KROW = D + 8;              // K row stride in LDS (16-bit elements)
  constexpr int VROW = kStage + 4;         // V^T row stride in LDS
  constexpr int KL = kStage * CH / kPfThreads;  // K chunks each thread stages
  constexpr int VPAIRS = CH * (kStage / 2);     // (chunk, token pair) items of V
  constexpr int KT = D / 32;               // k-steps of S^T = K Q^T
  constexpr int NDT = D / 16;              // d-tiles of O^T
  constexpr int KTOK_PER_WAVE = kWave / CH;         // K tokens one wave stages per load
  constexpr int VTOK_PER_WAVE = 2 * (kWave / CH);   // V tokens one wave stages
  static_assert(KL >= 1 && KL * kPfThreads == kStage * CH, "staging split");
  static_assert(VPAIRS <= kPfThreads, "one V pair per thread");
  static_assert(kBlockTokens % KTOK_PER_WAVE == 0 && kBlockTokens % VTOK_PER_WAVE == 0,
                "a wave's staged rows lie in one block");

  // V^T column of stage token tok in row r (a dim): 4-token column blocks
  // XOR-swizzled by bits 5-6 of the row, so that the staging stores (a wave
  // writes 16 rows 8 apart x 8 tokens) hit 64 distinct banks; 8-byte reads
  // of 4 consecutive tokens stay contiguous, and for the rows one d-tile
  // reads (r < 32 apart, same bits 5-6) the swizzle is a single constant.
  auto vt_col = [](int r, int tok) __attribute__((always_inline)) {
    return (((tok >> 2) ^ (2 * ((r >> 5) & 3))) << 2) | (tok & 3);
  };
  __shared__ __attribute__((aligned(16))) uint16_t lk[2][kStage * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t lv[2][D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int hgroups = p.num_kv_heads * p.hgroups_per_kv;
  const int wi = blockIdx.x / hgroups;
  const int hg = blockIdx.x - wi * hgroups;
  const int32_t* item = p.work + 6 * int64_t(wi);
  const int seq = item[0];
  const int tile = item[1];
  const int split = SPLIT ? item[4] : -1;
  const int kvh = hg / p.hgroups_per_kv;
  const int qh0 = kvh * p.group + (hg - kvh * p.hgroups_per_kv) * GW;
  const int L = p.context_lens[seq];
  const int qs = p.q_start[seq];
  const int T = p.q_start[seq + 1] - qs;
  const int C = L - T;
  const int t0 = tile * TQ;
  const int nblk = min((L + kBlockTokens - 1) / kBlockTokens, p.table_stride);
  const int32_t* trow = p.block_tables + int64_t(seq) * p.table_stride;
  const int64_t blk_stride = int64_t(p.num_kv_heads) * TILE;
  const char* kbase = p.k_cache + int64_t(kvh) * TILE;
  const char* vbase = p.v_cache + int64_t(kvh) * TILE;

  // query rows of this lane: group j holds row 16 j + n of the wave, i.e.
  // chunk token tq[j] = first + (16 j + n) / GW, head qh0 + n % GW
  const int h = qh0 + n % GW;
  const int wave_first = t0 + wave * TPW;
  int tq[RG], qpos[RG];
  bool row_ok[RG];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    tq[j] = wave_first + (16 * j + n) / GW;
    row_ok[j] = tq[j] < T;
    qpos[j] = C + tq[j];
  }
  const int wave_last = min(wave_first + TPW, T) - 1;  // < wave_first: no rows
  const int wg_last = min(t0 + TQ, T) - 1;
  const int wg_stages = (C + wg_last) / kStage + 1;
  const int s_begin = SPLIT ? item[2] : 0;
  const int s_end = SPLIT ? min(item[3], wg_stages) : wg_stages;
  const int wave_stages = wave_last >= wave_first ? (C + wave_last) / kStage + 1 : 0;
  const int mask_from = (C + wave_first) / kStage;  // first stage with a masked key

  u32x4 qb[RG][KT];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    const char* qrow = p.q + (int64_t(qs + (row_ok[j] ? tq[j] : 0)) * p.num_q_heads + h) * ROWB;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      qb[j][kt] = row_ok[j] ? *reinterpret_cast<const u32x4*>(qrow + (32 * kt + 8 * g) * 2)
                            : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- staging: global -> registers -> LDS ----------------------------------
  // Every wave's staged rows lie in one block, so the block index and the
  // buffer resource are wave-uniform.  The table entries come in chunks of
  // 64, one per lane of a register, read with v_readlane: a scalar load per
  // entry put a memory round trip (and a full wait) on every stage's path.
  u32x4 kr[KL];
  u32x4 vr0 = {0u, 0u, 0u, 0u}, vr1 = {0u, 0u, 0u, 0u};
  int tbl = -1, tbl_base = -kWave;  // entries tbl_base .. tbl_base + 63 (-1 past the sequence)
  auto table_entry = [&](int b) __attribute__((always_inline)) -> int {
    b = __builtin_amdgcn_readfirstlane(b);
    const int base = b & ~(kWave - 1);
    if (base != tbl_base) {  // wave-uniform; stages advance monotonically
      tbl_base = base;
      tbl = base + lane < nblk ? trow[base + lane] : -1;
    }
    return __builtin_amdgcn_readlane(tbl, b - base);
  };
  // the tile's byte offset as an unsigned 32 x 32 -> 64-bit product (the
  // launch checks that a block's stride fits 32 bits): two scalar multiplies
  auto tile_rsrc = [&](const char* base, int blk) __attribute__((always_inline)) {
    const bool ok = unsigned(blk) < unsigned(p.num_blocks);
    const uint64_t off = uint64_t(ok ? uint32_t(blk) : 0u) * uint32_t(blk_stride);
    return make_rsrc(base + off, ok ? TILE : 0);
  };
  // a block of the stage being loaded lies outside the pool (its keys are
  // masked when the stage is computed)
  bool bad_ld[2] = {false, false};
  bool bad_c[2] = {false, false};  // the same flags of the stage being computed
  float vmax = 0.f;                // largest |v| this thread staged (VCONV)
  auto load_stage = [&](int st) __attribute__((always_inline)) {
    const int ids[2] = {table_entry(st * 2), table_entry(st * 2 + 1)};
#pragma unroll
    for (int b = 0; b < 2; ++b) bad_ld[b] = !(unsigned(ids[b]) < unsigned(p.num_blocks));
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int idx = tid + i * kPfThreads;
      const int tok = idx / CH, ch = idx - (idx / CH) * CH;
      const int wtok = (wave * kWave + i * kPfThreads) / CH;  // first token of this wave's rows
      const auto rs = tile_rsrc(kbase, ids[wtok / kBlockTokens]);
      kr[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (tok % kBlockTokens) * ROWB + ch * 16, 0, 0));
    }
    if (wave * kWave < VPAIRS) {
      const int ch = tid % CH, tok = 2 * (tid / CH);
      const int wtok = 2 * (wave * kWave / CH);
      const auto rs = tile_rsrc(vbase, ids[wtok / kBlockTokens]);
      const int off = (tok % kBlockTokens) * ROWB + ch * 16;
      vr0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      vr1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + ROWB, 0, 0));
    }
  };
  auto store_stage = [&](int buf, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int idx = tid + i * kPfThreads;
      const int tok = idx / CH, ch = idx - (idx / CH) * CH;
      *reinterpret_cast<u32x4*>(&lk[buf][tok * KROW + ch * 8]) = kr[i];
    }
    if (wave * kWave < VPAIRS) {
      const int ch = tid % CH, tok = 2 * (tid / CH);
      uint32_t a[4] = {vr0.x, vr0.y, vr0.z, vr0.w};
      uint32_t b[4] = {vr1.x, vr1.y, vr1.z, vr1.w};
      if ((st + 1) * kStage > L) {  // the stage reaches past the context: those rows -> 0
        const int kp = st * kStage + tok;
        const uint32_t z0 = kp < L ? 0xFFFFFFFFu : 0u;
        const uint32_t z1 = kp + 1 < L ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] &= z0;
          b[i] &= z1;
        }
      }
      // dim e of the two tokens as one word (token tok low, tok + 1 high):
      // one byte permute per word; bf16 through fp32 to fp16 (exact below
      // 2^16 in magnitude, the largest magnitude kept for the overflow check)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t w;
        if constexpr (VCONV) {
          const uint32_t ua = (e & 1) ? (a[e >> 1] & 0xFFFF0000u) : (a[e >> 1] << 16);
          const uint32_t ub = (e & 1) ? (b[e >> 1] & 0xFFFF0000u) : (b[e >> 1] << 16);
          const f2 vv = {__uint_as_float(ua), __uint_as_float(ub)};
          vmax = fmaxf(vmax, fmaxf(fabsf(vv.x), fabsf(vv.y)));
          w = __builtin_bit_cast(uint32_t, __builtin_convertvector(vv, h2));
        } else {
          w = __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
        }
        *reinterpret_cast<uint32_t*>(&lv[buf][(ch * 8 + e) * VROW + vt_col(ch * 8 + e, tok)]) = w;
      }
    }
  };

  // ---- compute ----------------------------------------------------------------
  // Running maxima are kept in scaled base-2 units (score * scale * log2 e).
  const float c2 = p.scale_log2;
  float m[RG], lsum[RG];
  f4 o[RG][NDT];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    m[j] = kNegBig;
    lsum[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[j][dt] = f4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int buf, int st) __attribute__((always_inline)) {
    f4 sa[RG][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int j = 0; j < RG; ++j) sa[j][blk] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&lk[buf][(blk * 16 + n) * KROW + 32 * kt + 8 * g]);
#pragma unroll
        for (int j = 0; j < RG; ++j) sa[j][blk] = mfma_k32<DT>(a, qb[j][kt], sa[j][blk]);
      }
    }
    // blocks outside the pool contribute nothing (wave-uniform; flags taken
    // when the stage was loaded)
    const bool bad[2] = {bad_c[0], bad_c[1]};
    const bool masked = st >= mask_from || bad[0] || bad[1];
    u32x4 pb[RG], pl[RG];
    float s[RG][8], mxl[RG];
    bool moved = false;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[j][blk * 4 + v] = sa[j][blk][v];
      if (masked) {  // causal / context / pool mask (wave-uniform branch)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int kp = st * kStage + blk * 16 + 4 * g + v;
            if (bad[blk] || kp > qpos[j] || kp >= L) s[j][blk * 4 + v] = -INFINITY;
          }
      }
      mxl[j] = s[j][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mxl[j] = fmaxf(mxl[j], s[j][i]);
      // the running maximum moves only when a score exceeds it by more than
      // kRescaleSlack (weights stay <= 2^kRescaleSlack in between); the
      // lane's own 8 scores decide whether any of the row's can, so the
      // row's maximum over its four lanes is formed only in such a stage
      moved |= mxl[j] * c2 > m[j] + kRescaleSlack;
    }
    float alpha[RG] = {};
#pragma unroll
    for (int j = 0; j < RG; ++j) alpha[j] = 1.f;
    bool rescale = false;
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        const float mxs = max_over_lane_groups(mxl[j]) * c2;
        const float mn = mxs > m[j] + kRescaleSlack ? mxs : m[j];
        alpha[j] = __builtin_amdgcn_exp2f(m[j] - mn);
        rescale |= mn > m[j];
        m[j] = mn;
      }
    }
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const float mn = m[j];
      uint32_t ph[4], plo[4];
      float psum = 0.f;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][2 * q2], c2, -mn));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][2 * q2 + 1], c2, -mn));
        const f2 xx = {x0, x1};
        if constexpr (!PSPLIT) {
          // the normaliser sums the weights as rounded, the values the
          // products use: one dot product with (1, 1) per pair
          const h2 hp = __builtin_convertvector(xx, h2);
          ph[q2] = __builtin_bit_cast(uint32_t, hp);
          psum = __builtin_amdgcn_fdot2(hp, h2{1.f16, 1.f16}, psum, false);
        } else {
          psum += x0 + x1;
          const b2 hi = __builtin_convertvector(xx, b2);
          ph[q2] = __builtin_bit_cast(uint32_t, hi);
          plo[q2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(xx - __builtin_convertvector(hi, f2), b2));
        }
      }
      lsum[j] = lsum[j] * alpha[j] + psum;
      pb[j] = u32x4{ph[0], ph[1], ph[2], ph[3]};
      if constexpr (PSPLIT) pl[j] = u32x4{plo[0], plo[1], plo[2], plo[3]};
    }
    // rescale the accumulators only when some row's maximum moved
    if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
      for (int j = 0; j < RG; ++j)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[j][dt] *= alpha[j];
    }
    // V^T operands, each read one d-tile ahead of its products
    auto vt_operand = [&](int dt) __attribute__((always_inline)) -> u32x4 {
      const uint16_t* vrow = &lv[buf][(dt * 16 + n) * VROW];
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(vrow + vt_col(dt * 16, 4 * g));
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(vrow + vt_col(dt * 16, 16 + 4 * g));
      return u32x4{a0.x, a0.y, a1.x, a1.y};
    };
    // (two ahead where the registers allow: fp16 weights, no split records)
    constexpr int AHEAD = (!PSPLIT && !SPLIT) ? 2 : 1;
    u32x4 a_q[AHEAD];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) a_q[i] = vt_operand(i);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 a = a_q[dt % AHEAD];
      if (dt + AHEAD < NDT) a_q[dt % AHEAD] = vt_operand(dt + AHEAD);
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        o[j][dt] = mfma_k32<PVT>(a, pb[j], o[j][dt]);
        if constexpr (PSPLIT) o[j][dt] = mfma_k32<PVT>(a, pl[j], o[j][dt]);
      }
    }
  };

  if constexpr (!SPLIT) {
    // the whole tile, from stage 0 (kept apart from the stage-range loop
    // below: the compiler schedules this form better)
    load_stage(0);
    store_stage(0, 0);
    __syncthreads();
    for (int st = 0; st < wg_stages; ++st) {
      const int buf = st & 1;
      const bool more = st + 1 < wg_stages;
      bad_c[0] = bad_ld[0];
      bad_c[1] = bad_ld[1];
      if (more) load_stage(st + 1);
      if (st < wave_stages) compute(buf, st);
      if (more) store_stage(buf ^ 1, st + 1);
      __syncthreads();
    }
  } else {
    // a part: stages [s_begin, s_end) (never empty; the buffer parity is
    // the stage's own, so the loop has the same form as above)
    load_stage(s_begin);
    store_stage(s_begin & 1, s_begin);
    __syncthreads();
    for (int st = s_begin; st < s_end; ++st) {
      const int buf = st & 1;
      const bool more = st + 1 < s_end;
      bad_c[0] = bad_ld[0];
      bad_c[1] = bad_ld[1];
      if (more) load_stage(st + 1);
      if (st < wave_stages) compute(buf, st);
      if (more) store_stage(buf ^ 1, st + 1);
      __syncthreads();
    }
  }

  if constexpr (VCONV) {  // a staged V value fp16 cannot hold: the exact pass redoes this launch
    if (__builtin_amdgcn_ballot_w64(vmax >= 65536.f) && lane == 0)
      atomicMax(&g_v_overflow_launch, (unsigned long long)p.overflow_launch);
  }
  float lt[RG];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    lt[j] = lsum[j] + __shfl_xor(lsum[j], 16);
    lt[j] += __shfl_xor(lt[j], 32);
  }
  if (!SPLIT || split < 0) {
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      if (row_ok[j]) {
        const float inv = 1.f / lt[j];
        float* orow = p.out + (int64_t(qs + tq[j]) * p.num_q_heads + h) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<f4*>(orow + dt * 16 + 4 * g) = o[j][dt] * inv;
      }
    }
    return;
  }

  if constexpr (SPLIT) {
  // A part of a split tile: its (o, m, l) per row go to a record through
  // device-scope stores (visible to any XCD without cache flushes: o in
  // 16-byte sc1 stores, m and l as relaxed agent-scope atomics);
  // the part that takes the last ticket merges all parts:
  //   M = max m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
  if (split >= p.n_split) return;
  const int base = p.split_tab[2 * split];
  const int parts = p.split_tab[2 * split + 1];
  if (base < 0 || parts < 1 || base + parts > p.n_partials || item[5] >= parts) return;
  const int hgroups_total = hgroups;
  auto record = [&](int prt, int j) -> float* {
    const int row = wave * 16 * RG + 16 * j + n;
    return p.part + ((int64_t(base + prt) * hgroups_total + hg) * kPrefillTileRows + row) * p.rec_floats;
  };
  // the records of part prt of this (tile, head group): 128 rows, as a
  // buffer resource for the 16-byte device-scope accesses of o
  const int rec_bytes = p.rec_floats * 4;
  auto records = [&](int prt) -> __amdgpu_buffer_rsrc_t {
    return make_rsrc(p.part + (int64_t(base + prt) * hgroups_total + hg) * kPrefillTileRows * p.rec_floats,
                     kPrefillTileRows * rec_bytes);
  };
  const int row_off = (wave * 16 * RG + n) * rec_bytes + 16 * g;  // + 16 j rows + 64 dt
  {
    const __amdgpu_buffer_rsrc_t rs = records(item[5]);
#pragma unroll
    for (int j = 0; j < RG; ++j)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) store_device(rs, row_off + 16 * j * rec_bytes + 64 * dt, o[j][dt]);
  }
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    float* rec = record(item[5], j);
    if (g == 0) {
      __hip_atomic_store(rec + D, m[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(rec + D + 1, lt[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __shared__ int sm_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t* ticket = p.counters + int64_t(split) * hgroups_total + hg;
  if (tid == 0)
    sm_last = (__hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == parts - 1);
  __syncthreads();
  if (!sm_last) return;
  // every part's records were performed (agent-scope stores, waited for)
  // before its ticket was taken: order this workgroup's reads of them
  // after the ticket that counted the last part
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    float M = kNegBig;
    for (int prt = 0; prt < parts; ++prt)
      M = fmaxf(M, __hip_atomic_load(record(prt, j) + D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    f4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int prt = 0; prt < parts; ++prt) {
      const float* rec = record(prt, j);
      const float w = __builtin_amdgcn_exp2f(
          __hip_atomic_load(rec + D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - M);
      den = __builtin_fmaf(w, __hip_atomic_load(rec + D + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), den);
      const __amdgpu_buffer_rsrc_t rs = records(prt);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        acc[dt] += w * load_device(rs, row_off + 16 * j * rec_bytes + 64 * dt);
    }
    if (row_ok[j]) {
      const float inv = 1.f / den;
      float* orow = p.out + (int64_t(qs + tq[j]) * p.num_q_heads + h) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f4*>(orow + dt * 16 + 4 * g) = acc[dt] * inv;
    }
  }
    if (tid == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

typedef void (*PrefillFn)(const PrefillParams);

template <int DT, int D, bool SPLIT, bool EXACT>
PrefillFn pick_gw(int gw) {
  switch (gw) {
    case 1: return paged_prefill_kernel<DT, D, 1, SPLIT, EXACT>;
    case 2: return paged_prefill_kernel<DT, D, 2, SPLIT, EXACT>;
    case 4: return paged_prefill_kernel<DT, D, 4, SPLIT, EXACT>;
    case 8: return paged_prefill_kernel<DT, D, 8, SPLIT, EXACT>;
    case 16: return paged_prefill_kernel<DT, D, 16, SPLIT, EXACT>;
  }
  return nullptr;
}

template <int DT, int D, bool EXACT>
PrefillFn pick_split(int gw, bool split) {
  return split ? pick_gw<DT, D, true, EXACT>(gw) : pick_gw<DT, D, false, EXACT>(gw);
}

// exact: the bf16 exact pass (fp16 pools have one pass)
PrefillFn pick_prefill(int32_t dtype, int32_t head_dim, int gw, bool split, bool exact) {
  if (dtype == PKV_F16) {
    if (head_dim == 64) return pick_split<PKV_F16, 64, false>(gw, split);
    if (head_dim == 128) return pick_split<PKV_F16, 128, false>(gw, split);
  } else if (dtype == PKV_BF16) {
    if (head_dim == 64) return exact ? pick_split<PKV_BF16, 64, true>(gw, split) : pick_split<PKV_BF16, 64, false>(gw, split);
    if (head_dim == 128)
      return exact ? pick_split<PKV_BF16, 128, true>(gw, split) : pick_split<PKV_BF16, 128, false>(gw, split);
  }
  return nullptr;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_paged_prefill(const pkv_pool* pool, const void* q, float* out,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        const int32_t* block_tables, int32_t table_stride,
                                        const int32_t* context_lens, float scale, const int32_t* plan,
                                        const pkv_prefill_plan_info* info, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (!pool) return fail(PKV_E_BAD_ARG, "null pool");
  const pkv_pool_desc& d = pool->desc;
  if (!pool->k_cache || !pool->v_cache) return fail(PKV_E_BAD_ARG, "pool has no device K/V arrays");
  if (d.block_size != kBlockTokens) return fail(PKV_E_UNSUPPORTED, "device kernels take block_size 16 only");
  if (d.num_blocks < 1) return fail(PKV_E_BAD_ARG, "pool has no blocks");
  if (d.dtype != PKV_F16 && d.dtype != PKV_BF16)
    return fail(PKV_E_UNSUPPORTED, "paged prefill takes fp16 or bf16 pools");
  if (d.head_dim != 64 && d.head_dim != 128)
    return fail(PKV_E_UNSUPPORTED, "paged prefill takes head_dim 64 or 128");
  if (!info) return fail(PKV_E_BAD_ARG, "null plan info");
  // the running maxima are taken over scaled scores, which equals scaling
  // the maximum only for a positive scale
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PKV_E_BAD_ARG, "scale must be finite and > 0");
  if (int64_t(d.num_kv_heads) * kBlockTokens * d.head_dim * 2 > int64_t(UINT32_MAX))
    return fail(PKV_E_UNSUPPORTED, "a block of the pool spans more than 4 GiB");
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
    return fail(PKV_E_BAD_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / d.num_kv_heads;
  int gw = 1;
  while (gw < 16 && group % (2 * gw) == 0) gw *= 2;
  if (info->num_seqs != num_seqs || info->num_q_heads != num_q_heads ||
      info->num_kv_heads != d.num_kv_heads || info->tile_tokens != kPrefillTileRows / gw ||
      info->n_work < 0 || info->n_split < 0 || info->n_partials < 0)
    return fail(PKV_E_BAD_ARG, "plan info does not match this batch");
  if (table_stride < 1) return fail(PKV_E_BAD_ARG, "table_stride must be >= 1");
  if (int64_t(info->max_context_len) > int64_t(table_stride) * kBlockTokens)
    return fail(PKV_E_BAD_ARG, "a context is longer than its table can address");
  if (num_seqs == 0 || info->n_work == 0) return PKV_OK;
  if (!q || !out || !block_tables || !context_lens || !plan)
    return fail(PKV_E_BAD_ARG, "null device pointer");
  PrefillParams prm;
  prm.q = static_cast<const char*>(q);
  prm.out = out;
  prm.k_cache = static_cast<const char*>(pool->k_cache);
  prm.v_cache = static_cast<const char*>(pool->v_cache);
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  const size_t need = pkv_prefill_workspace_bytes(info, d.head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_E_BAD_ARG, "workspace too small: need " + std::to_string(need) + " bytes");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(workspace)) & 15)
    return fail(PKV_E_BAD_ARG, "q, out and workspace must be 16-byte aligned");
  prm.work = plan;
  prm.q_start = plan + 6 * int64_t(info->n_work);
  prm.split_tab = prm.q_start + num_seqs + 1;
  // records from the workspace's start, tickets at its end (as for decode:
  // launches of different shapes sharing one workspace sized for the
  // largest never put records where another launch's tickets are)
  const int64_t ticket_bytes =
      (int64_t(info->n_split) * d.num_kv_heads * (group / gw) * 4 + 255) / 256 * 256;
  prm.part = static_cast<float*>(workspace);
  prm.counters = need > 0 ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                       ((int64_t(workspace_bytes) - ticket_bytes) & ~int64_t(127)))
                          : nullptr;
  prm.rec_floats = int32_t(((int64_t(d.head_dim) + 2) * 4 + 127) / 128 * 32);
  prm.n_split = info->n_split;
  prm.n_partials = info->n_partials;
  prm.num_q_heads = num_q_heads;
  prm.num_kv_heads = d.num_kv_heads;
  prm.group = group;
  prm.hgroups_per_kv = group / gw;
  prm.table_stride = table_stride;
  prm.num_blocks = d.num_blocks;
  prm.scale_log2 = scale * kLog2eF;
  const int64_t grid = int64_t(info->n_work) * d.num_kv_heads * (group / gw);
  if (grid > INT32_MAX) return fail(PKV_E_BAD_ARG, "batch too large for one launch");
  const bool split = info->n_split > 0;
  prm.overflow_launch = 0;
  prm.gate_launch = 0;
  if (d.dtype == PKV_F16) {
    PrefillFn fn = pick_prefill(d.dtype, d.head_dim, gw, split, false);
    if (!fn) return fail(PKV_E_UNSUPPORTED, "no prefill kernel for this dtype / head_dim / group");
    hipLaunchKernelGGL(fn, dim3(uint32_t(grid)), dim3(kPfThreads), 0, static_cast<hipStream_t>(stream), prm);
    return launch_status("paged_prefill launch");
  }
  // bf16: the fast pass (V and weights in fp16), then the exact pass, which
  // runs only if the fast one met a V value of magnitude >= 2^16.
  // PKV_PREFILL_BF16_EXACT=1 runs the exact pass alone (read per call).
  PrefillFn fast = pick_prefill(d.dtype, d.head_dim, gw, split, false);
  PrefillFn exact = pick_prefill(d.dtype, d.head_dim, gw, split, true);
  if (!fast || !exact) return fail(PKV_E_UNSUPPORTED, "no prefill kernel for this dtype / head_dim / group");
  const char* ex = std::getenv("PKV_PREFILL_BF16_EXACT");
  if (ex && ex[0] == '1') {
    hipLaunchKernelGGL(exact, dim3(uint32_t(grid)), dim3(kPfThreads), 0, static_cast<hipStream_t>(stream), prm);
    return launch_status("paged_prefill launch");
  }
  static std::atomic<uint64_t> launches{0};
  const uint64_t id = launches.fetch_add(1, std::memory_order_relaxed) + 1;
  prm.overflow_launch = id;
  hipLaunchKernelGGL(fast, dim3(uint32_t(grid)), dim3(kPfThreads), 0, static_cast<hipStream_t>(stream), prm);
  const pkv_status st = launch_status("paged_prefill launch");
  if (st != PKV_OK) return st;
  prm.overflow_launch = 0;
  prm.gate_launch = id;
  hipLaunchKernelGGL(exact, dim3(uint32_t(grid)), dim3(kPfThreads), 0, static_cast<hipStream_t>(stream), prm);
  return launch_status("paged_prefill exact pass launch");
}
