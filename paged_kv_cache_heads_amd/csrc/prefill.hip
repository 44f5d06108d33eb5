// Varlen causal prefill attention with bf16 MFMA, over packed K/V or over the
// paged cache through a block table (prefix caching).
//
// What it computes: for sequence i with nq queries and nk keys (split by
// cu_seqlens_q / cu_seqlens_k), query j of head h attends with softmax weights
// scale * q.k to keys 0 .. nk - nq + j of kv head h / G (causal, queries
// aligned with the last keys), or to all nk keys (non-causal)
// (page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制": varlen prefill
// driven by cu_seqlens with an optional block_table for the prefix cache;
// page at bxzpzcl.cn/news/2159246, section 2.2.2: softmax(q kᵀ / sqrt(d)) v;
// page at hotelren.com/news/2273631, section 4.4: a cached prefix's KV is
// reused and only the remainder is computed).
//
// Design for gfx950 (the softmax, not the MFMA, is the scarce resource at
// head_dim 128: per score the MFMAs do 256 MACs while the vector units must
// scale, mask, exponentiate and convert it, so the kernel keeps that work to
// an FMA, an exp and half a convert per score):
// * One workgroup (4 waves) per (tile of 128/G query positions, kv head,
//   sequence): it covers all G query heads of the kv head, so every K/V tile
//   staged in LDS serves 128 query rows. The query tiles of one (sequence,
//   kv head) run back to back on one XCD (heaviest first), so their repeated
//   reads of the same K/V are served by that XCD's L2.
// * Each wave owns two 16-row subtiles (one head, 16 positions each).
// * Scores are computed transposed, Sᵀ = K Qᵀ, with v_mfma_f32_16x16x32_bf16:
//   K (row-major in LDS) is the A operand, Q (registers) the B operand. Each
//   lane then holds 16 keys of one query, so the row max needs a 2-step
//   exchange, and exp2(s - m) lands in registers already in the layout of the
//   B operand of Oᵀ = Vᵀ Pᵀ (the key order inside a 32-key step is permuted
//   the same way on both operands). V stays row-major in LDS and its Vᵀ
//   operand is read with ds_read_b64_tr_b16: inside each 16-lane group, lane
//   i returns element i % 4 of the 4-element segments addressed by lanes
//   4j + i / 4 (j = 0..3), so lane L pointing at V[4g + L/4][16 dt + 4 (L%4)]
//   yields V[4g + j][16 dt + L] for j = 0..3 -- four keys of one dim.
// * Row sums come out of the MFMA: a ninth 16-row output tile with a constant
//   all-ones A operand accumulates sum_k P[q][k] with the same rescaling as O,
//   and sums exactly the bf16-rounded P that the numerator uses.
// * The running maximum is rescaled lazily: O is rescaled only when a row's
//   maximum grows by more than 2^8, so p = 2^(s - m) stays below 2^8 and the
//   rescale is almost never taken after the first tiles.
// * LDS tiles are XOR-swizzled (no padding) so that the MFMA operand reads and
//   the staging writes are free of bank conflicts.
// * K and V tiles stream from global memory straight into LDS ring buffers
//   (global_load_lds_dwordx4: each lane's 16 bytes land at base + 16 *
//   lane), so later tiles are in flight during the current one's math with no
//   staging registers and one barrier per tile (a barrier that does not wait
//   for the loads still in flight). Tile addresses are a
//   scalar base plus a per-lane offset. Tiles that straddle the causal
//   diagonal or the sequence end are masked by selection (never by
//   multiplication), so stale cache bits cannot leak into the output; fully
//   visible tiles skip the mask.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mfma_tiles.h"

namespace pa {


constexpr int kPD = 128;        // head_dim
constexpr int kPThreads = 256;
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold, log2 units


// Workgroup barrier that does not drain outstanding loads (the tile DMA must
// stay in flight across it): this wave's LDS reads are complete, then
// s_barrier. The memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


template <int B>
using Buf = std::integral_constant<int, B>;

template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < N) {
    f(Buf<I>());
    static_for_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_from<0, N>(f); }


// Opaque re-definition of register values (no instruction is emitted).
template <int N>
__device__ __forceinline__ void launder(uint32_t (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}


// kRawMax: the scale is positive, so the running maximum is taken on raw
// scores and the scale folds into the exponent's FMA; otherwise scores are
// scaled first. BN: keys per tile, 64 (2 waves per SIMD) or 32 (half the
// score registers and LDS, 3 waves per SIMD: finer causal steps and more
// latency hiding for short sequences).
template <int G, bool kRawMax, int BN, bool kStore>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(BN == 32 ? 3 : 2, 8)))
void prefill_kernel(PrefillArgs a) {
  constexpr int kBN = BN;
  constexpr int KT = BN / 16;                // 16-key score tiles per tile
  constexpr int KK = BN / 32;                // 32-key steps of the PV product
  constexpr int DU = BN / 16;                // 1 KiB DMA instructions per wave per K (or V) tile
  constexpr int kTileBytes = BN * kPD * 2;   // one K or V tile
  // Buffers of [K tile | V tile]: 3 for 32-key tiles (48 KiB, three
  // workgroups per CU, tiles fetched two ahead), 2 for 64-key tiles (64 KiB,
  // two workgroups per CU, one ahead).
  // Each buffer is its own array and every access names it statically, so
  // the compiler can tell that reads of one buffer do not alias the DMA still
  // in flight into another and does not wait for that DMA before them.
  constexpr int STAGES = BN == 32 ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) char sbuf0[2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sbuf1[2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sbuf2[2 * kTileBytes];
  auto buffer = [&](auto b) -> char* {
    if constexpr (decltype(b)::value == 0) return sbuf0;
    else if constexpr (decltype(b)::value == 1) return sbuf1;
    else return sbuf2;
  };

  constexpr int QP = 128 / G;  // query positions per workgroup
  constexpr int PB = QP / 16;  // 16-position subtiles per head
  // Work item of this workgroup. Workgroup ids are dealt to the 8 XCDs
  // round-robin (id % 8) and each XCD has its own L2, so XCD x takes the
  // contiguous slice x of the items, ordered kv head first. Under the causal
  // mask a query tile costs in proportion to its index, so within a head the
  // items go heaviest first: the query tiles are taken in pairs from the
  // last one down (tiles T-1 and T-2 of every sequence, then T-3 and T-4 of
  // every sequence, ...; with T odd, tile 0 alone at the end), sequence by
  // sequence within a pair. The long tiles then start in the first wave of
  // workgroups and the short ones fill the tail, while the two tiles of a
  // pair still read the same sequence's K/V through the XCD's L2.
  const int64_t item = (int64_t)(blockIdx.x & 7) * a.items_per_xcd + (blockIdx.x >> 3);
  const int64_t per_head = (int64_t)a.num_q_tiles * a.num_seqs;
  if (item >= (int64_t)a.num_kv_heads * per_head) return;
  const int kvh = (int)(item / per_head);
  const int64_t r = item - (int64_t)kvh * per_head;
  const int64_t pair_items = 2 * (int64_t)a.num_seqs;
  const int64_t paired = pair_items * (a.num_q_tiles / 2);
  int seq, qtile;
  if (r < paired) {
    const int pair = (int)(r / pair_items);
    const int w = (int)(r - pair * pair_items);
    seq = w >> 1;
    qtile = a.num_q_tiles - 1 - 2 * pair - (w & 1);
  } else {
    seq = (int)(r - paired);
    qtile = 0;
  }
  const int q_beg = a.cu_seqlens_q[seq];
  const int nq = a.cu_seqlens_q[seq + 1] - q_beg;
  const int k_beg = a.cu_seqlens_k[seq];
  const int nk = a.cu_seqlens_k[seq + 1] - k_beg;
  const int q0 = qtile * QP;
  if (q0 >= nq) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int shift = nk - nq;  // causal: query j sees keys <= shift + j

  // ---- this lane's two query rows ----
  int head[2], qpos[2], lim[2];
  uint4 qop[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int st = wave * 2 + u;
    head[u] = kvh * G + st / PB;
    qpos[u] = q0 + (st % PB) * 16 + col;
    lim[u] = a.causal ? shift + qpos[u] : nk - 1;
    const int qc = min(qpos[u], nq - 1);
    const bf16_t* qr = a.q + (int64_t)(q_beg + qc) * a.q_token_stride + (int64_t)head[u] * kPD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qop[u][ks] = load16(qr + ks * 32 + 8 * g);
  }

  // keys this workgroup needs, and the first key some row cannot see
  const int q_last = min(q0 + QP, nq) - 1;
  const int k_end = a.causal ? min(nk, shift + q_last + 1) : nk;
  const int full_below = a.causal ? min(nk, shift + q0 + 1) : nk;  // keys < this are visible to every row
  const int ntiles = k_end > 0 ? (k_end + kBN - 1) / kBN : 0;

  // Oᵀ accumulators: 8 tiles of 16 dims + the row-sum tile
  f32x4_t oacc[2][9];
  float m[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    m[u] = kNegBig;
#pragma unroll
    for (int dt = 0; dt < 9; ++dt) oacc[u][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Tile staging: DMA instruction u (u < DU) of wave w fills the 1 KiB of
  // rows 16u + 4w .. 16u + 4w + 3; lane i supplies row 16u + 4w + i / 16,
  // physical chunk i % 16, i.e. the logical chunk that the swizzle maps
  // there. The swizzle only depends on the row mod 16, which is the same for
  // every u, so one per-lane offset serves all instructions of a tile and the
  // rest of each address is uniform.
  const int64_t kstride = a.block_table ? (int64_t)a.num_kv_heads * kPD : a.k_token_stride;
  const int64_t vstride = a.block_table ? (int64_t)a.num_kv_heads * kPD : a.v_token_stride;
  const int srow0 = 4 * wave + (lane >> 4);  // row of instruction 0; + 16u for instruction u
  const uint32_t kofs = (uint32_t)(srow0 * kstride * 2) + (((lane & 15) ^ (srow0 & 15)) << 4);
  const uint32_t vofs = (uint32_t)(srow0 * vstride * 2) + (((lane & 15) ^ ((srow0 & 7) << 1)) << 4);

  // K operand reads: row kt * 16 + col, logical chunk 4 ks + g (swizzled by col).
  uint32_t koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = k_off(col, ks * 4 + g);
  uint32_t voff[8];
  {
    const int trow = 4 * g + (col >> 2), tq = col & 3;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) voff[dt] = v_off(trow, 2 * dt + (tq >> 1)) + (tq & 1) * 8;
  }

  // Block-table entries of this sequence, 64 at a time: lane i holds entry
  // tbase + i (entries past the ones the sequence uses read as 0).
  const int nblk = a.block_table ? min(a.max_blocks_per_seq, (nk + a.block_size - 1) / max(a.block_size, 1)) : 0;
  int tbase = 0, tentry = 0;
  // The load is waited for where it is issued (rarely: every 64 blocks), so
  // that the compiler's wait bookkeeping never sees the entry pending at a
  // later use; otherwise it drains all tile DMA in flight before every
  // block lookup.
  auto load_table = [&](int base) {
    tbase = base;
    tentry = base + lane < nblk ? a.block_table[(int64_t)seq * a.max_blocks_per_seq + base + lane] : 0;
    wait_vmem_le<0>();
  };
  if (a.block_table) load_table(0);
  int iblk = 0, ioff = 0;  // block and offset of the next tile to issue (tiles never straddle a block)

  auto issue_tile = [&](int t0, char* kdst) {
    int64_t krow0, vrow0;
    if (a.block_table == nullptr) {
      krow0 = (int64_t)(k_beg + t0) * kstride;
      vrow0 = (int64_t)(k_beg + t0) * vstride;
    } else {
      if (iblk - tbase >= 64) load_table(iblk);
      const int blk = __builtin_amdgcn_readlane(tentry, iblk - tbase);
      krow0 = vrow0 = ((int64_t)blk * a.block_size + ioff) * kstride;
      ioff += kBN;
      if (ioff == a.block_size) ioff = 0, ++iblk;
    }
    const char* kb = reinterpret_cast<const char*>(a.k + krow0 + kvh * kPD);
    const char* vb = reinterpret_cast<const char*>(a.v + vrow0 + kvh * kPD);
    char* vdst = kdst + kTileBytes;
    const int last = nk - 1 - t0;  // rows past it are clamped to it (t0 < nk, so last >= 0)
    if constexpr (kStore && BN == 64) {  // the fused store through a table always runs 64-key tiles
      if (a.block_table != nullptr && t0 + kBN > shift) {
        // Fused store through a block table: keys at positions >= shift are
        // the new tokens, not in the cache yet; their rows come from k_new /
        // v_new (row q_beg + position - shift). A tile that starts below shift
        // takes its first rows from the cache as above (two passes, each lane
        // in the one that holds its row; extra instructions only make the
        // tile waits stricter).
        const int nrow0 = max(t0 - shift, 0);  // first new-token row the tile needs
        const char* nkb = reinterpret_cast<const char*>(a.k_new + (int64_t)(q_beg + nrow0) * a.k_new_stride + kvh * kPD);
        const char* nvb = reinterpret_cast<const char*>(a.v_new + (int64_t)(q_beg + nrow0) * a.v_new_stride + kvh * kPD);
        const uint32_t kch = ((lane & 15) ^ (srow0 & 15)) << 4;
        const uint32_t vch = ((lane & 15) ^ ((srow0 & 7) << 1)) << 4;
#pragma unroll
        for (int u = 0; u < DU; ++u) {
          const int row = min(srow0 + 16 * u, last);
          const int o = (16 * u + 4 * wave) * 256;
          const int nr = t0 + row - shift - nrow0;  // row within the tile's new-token rows (< kBN)
          if (nr >= 0) {
            __builtin_amdgcn_global_load_lds(nkb + (uint32_t)(nr * a.k_new_stride * 2) + kch,
                                             (lds_void_t*)(kdst + o), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(nvb + (uint32_t)(nr * a.v_new_stride * 2) + vch,
                                             (lds_void_t*)(vdst + o), 16, 0, 0);
          } else {
            __builtin_amdgcn_global_load_lds(kb + (uint32_t)(row * kstride * 2) + kch, (lds_void_t*)(kdst + o),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(vb + (uint32_t)(row * vstride * 2) + vch, (lds_void_t*)(vdst + o),
                                             16, 0, 0);
          }
        }
        return;
      }
    }
    // byte offsets from the tile's first row (below 2^31: checked on the host);
    // a clamped row keeps its lane's swizzled chunk, selected without a branch
    const uint32_t kcl = (uint32_t)(last * kstride * 2) + (((lane & 15) ^ (srow0 & 15)) << 4);
    const uint32_t vcl = (uint32_t)(last * vstride * 2) + (((lane & 15) ^ ((srow0 & 7) << 1)) << 4);
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const bool clamp = srow0 + 16 * u > last;
      const uint32_t ko = clamp ? kcl : (uint32_t)(16 * u * kstride * 2) + kofs;
      const uint32_t vo = clamp ? vcl : (uint32_t)(16 * u * vstride * 2) + vofs;
      const int o = (16 * u + 4 * wave) * 256;
      __builtin_amdgcn_global_load_lds(kb + ko, (lds_void_t*)(kdst + o), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vb + vo, (lds_void_t*)(vdst + o), 16, 0, 0);
    }
  };

  // Softmax in log2 units: p = 2^(c*s - c*m).
  const float c = kRawMax ? a.scale_log2e : 1.f;
  const float tau = kRescaleLog2 / c;  // threshold in score units
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 1.0 pairs

  // Tiles are issued STAGES - 1 ahead, tile t into buffer t % STAGES; loads
  // complete in issue order, so K/V(t) has landed once at most the following
  // tile's 2 * DU instructions are outstanding.
  if (ntiles > 0) issue_tile(0, buffer(Buf<0>()));
  if constexpr (STAGES > 2)
    if (ntiles > 1) issue_tile(kBN, buffer(Buf<1>()));
  auto step = [&](int tile, auto rb) {
    constexpr int RB = decltype(rb)::value;
    const int t0 = tile * kBN;
    if (STAGES > 2 && tile + 1 < ntiles) wait_vmem_le<2 * DU>(); else wait_vmem_le<0>();
    barrier_keep_loads();  // everyone's tile is in; everyone finished tile - 1
    // The next DMA goes out before the score MFMAs with two stages (it has one
    // tile to land), after them with three (two tiles to land), so that its
    // issue overlaps the MFMAs in flight.
    if (STAGES == 2 && tile + 1 < ntiles) issue_tile(t0 + kBN, buffer(Buf<(RB + 1) % STAGES>()));
    const char* sK = buffer(rb);
    const char* sV = sK + kTileBytes;
    // Re-define the per-lane LDS offsets at every step, so that the compiler
    // adds them to this step's buffer here instead of keeping a hoisted
    // address per buffer live across the loop.
    launder(koff);
    launder(voff);

    // ---- Sᵀ = K Qᵀ for both subtiles (8 independent accumulators per k-step) ----
    f32x4_t sacc[2][KT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) sacc[u][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (BN == 32) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint4 kop[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) kop[kt] = *reinterpret_cast<const uint4*>(sK + kt * 16 * 256 + koff[ks]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          sacc[0][kt] = mfma16x16x32(kop[kt], qop[0][ks], sacc[0][kt]);
          sacc[1][kt] = mfma16x16x32(kop[kt], qop[1][ks], sacc[1][kt]);
        }
      }
    } else {
      // K operand read j = ks * KT + kt feeds the two MFMAs of (ks, kt); the
      // reads are scheduled six ahead of their MFMAs (mask 0x100: LDS reads,
      // 0x008: MFMA), where the compiler's own order drains the LDS queue
      // before every k-step.
      constexpr int NR = 4 * KT;
      uint4 kop[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) kop[j] = *reinterpret_cast<const uint4*>(sK + (j % KT) * 16 * 256 + koff[j / KT]);
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        sacc[0][j % KT] = mfma16x16x32(kop[j], qop[0][j / KT], sacc[0][j % KT]);
        sacc[1][j % KT] = mfma16x16x32(kop[j], qop[1][j / KT], sacc[1][j % KT]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int j = 0; j < NR - 6; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
    }

    if (STAGES > 2 && tile + STAGES - 1 < ntiles)
      issue_tile(t0 + (STAGES - 1) * kBN, buffer(Buf<(RB + STAGES - 1) % STAGES>()));

    // ---- softmax numerators (each lane: one query, keys kt*16 + 4g + i) ----
    const bool need_mask = (t0 + kBN > full_below);
    uint4 pop[2][KK];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float x[KT][4];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[kt][i] = kRawMax ? sacc[u][kt][i] : sacc[u][kt][i] * a.scale_log2e;
      if (need_mask) {
        // key t0 + kt*16 + 4g + i is visible iff kt*16 + i <= rel
        const int rel = min(lim[u], nk - 1) - t0 - 4 * g;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[kt][i] = (kt * 16 + i <= rel) ? x[kt][i] : -INFINITY;
      }
      // row max: this lane's scores (a chain of 3-input maxima), then the
      // lanes holding the same query (lane ^ 16, lane ^ 32)
      float mx = fmaxf(fmaxf(x[0][0], x[0][1]), x[0][2]);
#pragma unroll
      for (int e = 3; e + 1 < 4 * KT; e += 2) mx = fmaxf(fmaxf(mx, x[e / 4][e % 4]), x[(e + 1) / 4][(e + 1) % 4]);
      mx = fmaxf(mx, x[KT - 1][3]);
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      if (__ballot(mx > m[u] + tau)) {
        const float mnew = fmaxf(m[u], mx);
        if (tile != 0) {  // on the first tile the accumulators are still zero
          const float alpha = fast_exp2((m[u] - mnew) * c);
#pragma unroll
          for (int dt = 0; dt < 9; ++dt) oacc[u][dt] *= alpha;
        }
        m[u] = mnew;
      }
      const float mc = m[u] * c;
      float p[KT][4];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[kt][i] = fast_exp2(fmaf(x[kt][i], c, -mc));
      // B operand of Oᵀ = Vᵀ Pᵀ for 32-key step kk: slots 0..3 <- tile 2kk, slots 4..7 <- tile 2kk+1
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        pop[u][kk].x = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
        pop[u][kk].y = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
        pop[u][kk].z = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
        pop[u][kk].w = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
      }
    }

    // ---- Oᵀ += Vᵀ Pᵀ, and the row sums (16 independent accumulators per k-step) ----
    // Read pair (kk, dt): keys 32 kk + 0..15 and 16..31, dims 16 dt .. 16 dt + 15.
    // The LDS pointer is derived from this step's own stage array, so the
    // compiler can tell these reads from the DMA in flight into the others.
    typedef __attribute__((address_space(3))) const char lds_char_t;
    lds_char_t* vl = (lds_char_t*)sV;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vl + kk * 32 * 256 + voff[dt]));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vl + (kk * 32 + 16) * 256 + voff[dt]));
        const v2i_t l2 = __builtin_bit_cast(v2i_t, lo), h2 = __builtin_bit_cast(v2i_t, hi);
        const uint4 vop = make_uint4(l2.x, l2.y, h2.x, h2.y);
        oacc[0][dt] = mfma16x16x32(vop, pop[0][kk], oacc[0][dt]);
        oacc[1][dt] = mfma16x16x32(vop, pop[1][kk], oacc[1][dt]);
        if (dt == 7) {
          oacc[0][8] = mfma16x16x32(ones, pop[0][kk], oacc[0][8]);
          oacc[1][8] = mfma16x16x32(ones, pop[1][kk], oacc[1][8]);
        }
      }
    if constexpr (BN == 64) {
      // 64-key tiles: keep four read pairs ahead of their MFMAs (mask 0x100:
      // LDS reads, 0x008: MFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int j = 0; j < 12; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 12, 1);
    }
  };
  for (int tile = 0; tile < ntiles; tile += STAGES) {
    step(tile, Buf<0>());
    if (tile + 1 < ntiles) step(tile + 1, Buf<1>());
    if constexpr (STAGES > 2)
      if (tile + 2 < ntiles) step(tile + 2, Buf<2>());
  }

  // ---- fused store, first half: load this item's new tokens' K and V rows of kv head kvh ----
  // New token j of the sequence (one per query) is row q_beg + j of k_new / v_new. The item of query
  // tile j / QP stores it, so every row is written once. The rows were just read by this item's last
  // tiles, so the loads are served by L2; they are issued here so that their latency overlaps the
  // output epilogue. 32 vectors of 16 bytes per token (K then V).
  constexpr int kVecs = kStore ? QP * 32 / kPThreads : 1;  // vectors per thread
  uint4 sval[kVecs];
  int sslot[kVecs];
  if constexpr (kStore) {
    const int ntok = min(QP, nq - q0);
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const int v = tid + i * kPThreads;
      const int j = v >> 5, c = v & 31;
      sslot[i] = -1;
      if (j < ntok) {
        const int64_t row = q_beg + q0 + j;
        const int s = a.slot_mapping[row];
        const uint16_t* src = (c >= 16 ? a.v_new + row * a.v_new_stride : a.k_new + row * a.k_new_stride) +
                              kvh * kPD + (c & 15) * 8;
        sval[i] = load16(src);
        sslot[i] = s >= 0 && s < a.store_capacity ? s : -1;
      }
    }
  }

  // ---- epilogue: normalise and write the rows that exist ----
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (qpos[u] >= nq) continue;
    const float ls = oacc[u][8][0];
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    bf16_t* orow = a.out + ((int64_t)(q_beg + qpos[u]) * a.num_q_heads + head[u]) * kPD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(oacc[u][dt][0] * inv, oacc[u][dt][1] * inv);
      w.y = pack_bf16x2(oacc[u][dt][2] * inv, oacc[u][dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * g) = w;
    }
  }

  // ---- fused store, second half: the rows to their slots ----
  if constexpr (kStore) {
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      if (sslot[i] >= 0) {
        const int c = (tid + i * kPThreads) & 31;
        uint16_t* cache = c >= 16 ? a.v_cache_out : a.k_cache_out;
        store16_nt(cache + (int64_t)sslot[i] * a.num_kv_heads * kPD + kvh * kPD + (c & 15) * 8, sval[i]);
      }
    }
  }
}

template <int G, int BN, bool kStore>
static void launch_prefill_gbs(const PrefillArgs& a, hipStream_t stream) {
  // one workgroup per work item, 8 XCD slices of items_per_xcd each
  dim3 grid((unsigned)(8 * a.items_per_xcd));
  if (a.scale_log2e > 0.f)
    prefill_kernel<G, true, BN, kStore><<<grid, dim3(kPThreads), 0, stream>>>(a);
  else
    prefill_kernel<G, false, BN, kStore><<<grid, dim3(kPThreads), 0, stream>>>(a);
}

template <int G, int BN>
static void launch_prefill_gb(const PrefillArgs& a, hipStream_t stream) {
  if (a.slot_mapping)
    launch_prefill_gbs<G, BN, true>(a, stream);
  else
    launch_prefill_gbs<G, BN, false>(a, stream);
}

template <int G>
static hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t stream) {
  // the fused store through a block table runs 64-key tiles (its per-row
  // source choice does not fit the 32-key kernel's registers)
  if (prefill_key_tile(a.max_seqlen_k) == 32 && !(a.slot_mapping && a.block_table))
    launch_prefill_gb<G, 32>(a, stream);
  else
    launch_prefill_gb<G, 64>(a, stream);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t stream) {
  if (a.num_seqs == 0 || a.num_q_tiles == 0) return hipSuccess;
  switch (group) {
    case 1: return launch_prefill_g<1>(a, stream);
    case 2: return launch_prefill_g<2>(a, stream);
    case 4: return launch_prefill_g<4>(a, stream);
    case 8: return launch_prefill_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
