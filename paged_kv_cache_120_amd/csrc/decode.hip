// Paged decode attention for gfx950 (CDNA4, wave64).
//
// What it computes: vLLM book ch.4 "PagedAttention：虚拟内存的启示", §4.5
// (walk the block table in logical order, read each physical block) and §4.6
// (online softmax; fp32 statistics and accumulators).  For sequence i and
// query head h, over exactly context_len tokens:
//   out[i,h] = sum_t softmax_t(scale <q[i,h], K_t>) V_t,  kv head = h / g.
//
// A workgroup (4 or 8 waves) processes a token range [t0, t1) of one (kv head,
// sequence) and serves all g query heads of that kv head, so each K/V byte is
// fetched from HBM once and reused g times.  Two range bodies exist:
//   ValuPath      -- vector ALU, dot products reduced with DPP (g = 1, 2,
//                    and 4 at head size 64);
//   MfmaSplitPath -- both contractions on the matrix cores (g = 8, g = 4 at
//                    head size 128, and 16 columns of (query token, head)
//                    or (member, head) pairs).
// Kernels driving them:
//   partition_kernel -- one range per workgroup: a whole sequence (single
//                       pass) or one fixed partition (split-KV);
//   balanced_kernel  -- a grid sized to the workgroups the chip holds at
//                       once; each takes an equal slice of all the KV work
//                       (possibly several ranges); the last range of a split
//                       pair to finish merges its partial states;
//   reduce_kernel    -- merges the fixed partitions of split-KV with the
//                       §4.6 recurrence, many partitions in flight per
//                       workgroup.
//
// Common to both bodies: K/V rows are read with 16-byte buffer loads whose
// resource is rebased per physical block (64-bit base in SGPRs) with a record
// count that ends at the last valid token, so slots past context_len are
// never fetched (padding may hold Inf/NaN).  The loads are non-temporal: each
// byte is used once per step.  Block ids for a 64-block window come from one
// vector load per wave and are broadcast with v_readlane.  Scores are kept in
// base-2 units (x log2 e) so every exponential is one v_exp_f32.
#include <type_traits>

#include "common.h"
#include "decode.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online softmax with a lazy reference (base-2 units): scores are
// exponentiated against a reference that moves only when a batch max
// exceeds it by more than kSlack, so weights stay <= 2^kSlack and the
// rescale of the accumulators is skipped for almost every batch; the state
// is brought to the true max once, at the end of a range.
constexpr float kSlack = 8.f;
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;

// Physical block ids of logical blocks [win, win + 64) of one sequence, one
// per lane; entries at or past `end` are never read from the table.
struct BlockWindow {
  const int* bt;
  int end;
  int win;
  int ids;
  __device__ void init(const int* row, int first, int end_, int lane) {
    bt = row;
    end = end_;
    win = first;
    ids = (win + lane < end) ? bt[win + lane] : 0;
  }
  // make the window hold logical blocks first .. last (last - first < 64)
  __device__ void cover(int first, int last, int lane) {
    if (last >= win + 64) {
      win = first;
      ids = (win + lane < end) ? bt[win + lane] : 0;
    }
  }
  __device__ int block(int lb) const {
    return __builtin_amdgcn_readlane(ids, lb - win);
  }
};

// Buffer resource over the valid rows of logical block lb of one head:
// record count = valid tokens x row stride (0 for a block past the end or an
// id outside the pool, which then reads as zeros without touching memory).
template <int B>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(
    const char* head_base, int blk, int lb, int t1, uint32_t row_stride,
    uint64_t blk_bytes, int num_blocks) {
  int valid = t1 - lb * B;
  valid = valid < B ? valid : B;
  const bool ok = valid > 0 && (unsigned)blk < (unsigned)num_blocks;
  return make_rsrc(head_base + (ok ? (uint64_t)blk * blk_bytes : 0),
                   ok ? (uint32_t)valid * row_stride : 0u);
}

// Fused append: store this step's K/V row of head kvh (token `last` of the
// sequence) into its slot and record the slot.  Called by the one range
// that holds token `last`; lanes 0 .. D/8-1 of wave 0 each move 8 elements:
// 16 bytes bit for bit into an fp16 pool, or their 8 e4m3 codes (quantised
// as pa_cache_write_fp8 does) into an fp8 pool.  A slot outside the pool is
// skipped, as in the cache write.
template <int D, int B, int EB>
__device__ __forceinline__ void append_token(const DecodeArgs& a, int kvh,
                                             int seq, int last) {
  if (threadIdx.x >= D / 8) return;
  const int blk = a.block_tables[(size_t)seq * a.max_blocks_per_seq + last / B];
  const long long slot = (long long)blk * B + last % B;
  const bool ok = blk >= 0 && blk < a.num_blocks;
  if (kvh == 0 && threadIdx.x == 0 && a.slot_out)
    a.slot_out[seq] = ok ? (int)slot : -1;
  if (!ok) return;
  const size_t src = ((size_t)seq * a.num_kv_heads + kvh) * D + threadIdx.x * 8;
  const size_t dst = ((size_t)slot * a.num_kv_heads * D + (size_t)kvh * D +
                      threadIdx.x * 8) * EB;
  char* kc = const_cast<char*>(a.key_cache);
  char* vc = const_cast<char*>(a.value_cache);
  const u32x4 k = *reinterpret_cast<const u32x4*>(a.new_key + src);
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.new_value + src);
  if constexpr (EB == 2) {
    *reinterpret_cast<u32x4*>(kc + dst) = k;
    *reinterpret_cast<u32x4*>(vc + dst) = v;
  } else {
    *reinterpret_cast<u32x2*>(kc + dst) = f16x8_to_fp8x8(k, a.inv_k_scale);
    *reinterpret_cast<u32x2*>(vc + dst) = f16x8_to_fp8x8(v, a.inv_v_scale);
  }
}

// Final cross-wave merge.  Each wave left (m, l) per head and acc[head][d] in
// LDS; every thread folds one (head, channel) and hands the result to `sink`
// as (head in group, channel, max in base-2 units, sum, unnormalised out).
template <int D, int G, class Smem, class Sink>
__device__ __forceinline__ void merge_waves(Smem& sm, Sink& sink) {
  constexpr int W = sizeof(sm.m) / sizeof(sm.m[0]);    // waves of the body
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int gi = idx / D;
    const int d = idx % D;
    float mx = sm.m[0][gi];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, sm.m[w][gi]);
    const float sh = mx == -INFINITY ? 0.f : mx;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = fast_exp2(sm.m[w][gi] - sh);
      L += sm.l[w][gi] * f;
      O += sm.acc[w][gi][d] * f;
    }
    sink(gi, d, mx, L, O);
  }
  __syncthreads();    // LDS free for the next range
}

// One load of 8 cached elements: 16 bytes of fp16 (EB = 2) or 8 bytes of
// e4m3 codes (EB = 1), kept in that form until used, then widened to fp16.
template <int EB, int AUX = kLoadNt>
struct KvLoad {
  using type = u32x4;
  __device__ static type load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return load16<AUX>(r, off);
  }
};
template <int AUX>
struct KvLoad<1, AUX> {
  using type = u32x2;
  __device__ static type load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return load8<AUX>(r, off);
  }
};
__device__ __forceinline__ u32x4 widen(u32x4 v) { return v; }
__device__ __forceinline__ u32x4 widen(u32x2 v) { return fp8x8_to_f16x8(v); }

// ---------------------------------------------------------------------------
// Vector-ALU range body
// ---------------------------------------------------------------------------
//
// A 16-byte load per lane covers one token row of one head (D/8 lanes per
// row), so one load instruction reads whole 128-byte lines.  A wave batch is
// NJ loads of K and NJ of V per lane in flight; the W waves take batches
// round-robin.  Each row group (one token of a load) keeps its own online
// softmax state (m, l, acc[8] per head, replicated in the row): the dot
// product is reduced across the row with four DPP adds (bitwise identical in
// every lane) and everything else is lane-local until the end, where row
// groups merge with cross-lane shuffles and waves through LDS.
template <int D, int B, int G, int NJ, int EB = 2, int W = kWaves>
struct ValuPath {
  static constexpr int kWavesWG = W;      // waves per workgroup
  static constexpr int LPR = D / 8;       // lanes per token row
  static constexpr int RPI = 64 / LPR;    // token rows per wave load
  static constexpr int TB = RPI * NJ;     // tokens per wave batch
  // waves per SIMD the balanced kernel is register-limited to (1: no
  // limit); groups of 1 and 4 fit in 128 VGPRs, 4 waves, without spilling
  static constexpr int kMinWaves = (G == 1 || G == 4) ? 4 : 1;
  static_assert(B % RPI == 0, "a load must not straddle two blocks");

  struct Smem {
    float acc[W][G][D];
    float m[W][G];
    float l[W][G];
  };

  // t0 must be a multiple of RPI (callers pass multiples of 16).  `last` is
  // the position of this step's appended token if it lies in [t0, t1) and
  // the step is fused, else -1.
  template <class Sink>
  __device__ static void run(const DecodeArgs& a, Smem& sm, int kvh, int seq,
                             int t0, int t1, int last, Sink& sink) {
    const int H = a.num_heads;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane / LPR;
    const int c = lane % LPR;
    if (last >= 0) append_token<D, B, EB>(a, kvh, seq, last);

    u32x4 qv[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
      qv[gi] = *reinterpret_cast<const u32x4*>(
          a.query + ((size_t)seq * H + (size_t)kvh * G + gi) * D + c * 8);

    BlockWindow bw;
    bw.init(a.block_tables + (size_t)seq * a.max_blocks_per_seq, t0 / B,
            (t1 + B - 1) / B, lane);
    const uint32_t row_stride = (uint32_t)a.num_kv_heads * D * EB;
    const uint64_t blk_bytes = (uint64_t)B * row_stride;
    const char* kbase = a.key_cache + (size_t)kvh * D * EB;
    const char* vbase = a.value_cache + (size_t)kvh * D * EB;
    // fp8 pools: K's scale folds into the score scale, V's into the output
    const float sl2 = a.scale * kLog2e * (EB == 1 ? a.k_scale : 1.f);

    // m: the reference the state is kept relative to; mt: the true max
    float m[G], mt[G], l[G], acc[G][8];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      m[gi] = -INFINITY;
      mt[gi] = -INFINITY;
      l[gi] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
    }

    // loads of one batch into (kk, vv), including the appended token's row
    using Raw = typename KvLoad<EB>::type;
    auto issue = [&](int base, Raw (&kk)[NJ], Raw (&vv)[NJ]) {
      bw.cover(base / B, (base + TB - 1) / B, lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int tok0 = base + j * RPI;   // wave-uniform
        const int lb = tok0 / B;
        const int blk = bw.block(lb);
        const uint32_t off = (uint32_t)(tok0 % B + r) * row_stride + c * 8 * EB;
        const __amdgpu_buffer_rsrc_t rk = block_rsrc<B>(
            kbase, blk, lb, t1, row_stride, blk_bytes, a.num_blocks);
        const __amdgpu_buffer_rsrc_t rv = block_rsrc<B>(
            vbase, blk, lb, t1, row_stride, blk_bytes, a.num_blocks);
        kk[j] = KvLoad<EB>::load(rk, off);
        vv[j] = KvLoad<EB>::load(rv, off);
      }
      if (last >= 0 && base + TB > last) {   // the appended row
        const size_t src = ((size_t)seq * a.num_kv_heads + kvh) * D + c * 8;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (base + j * RPI + r == last) {
            const u32x4 nk = *reinterpret_cast<const u32x4*>(a.new_key + src);
            const u32x4 nv = *reinterpret_cast<const u32x4*>(a.new_value + src);
            if constexpr (EB == 2) {
              kk[j] = nk;
              vv[j] = nv;
            } else {   // the codes the append stores
              kk[j] = f16x8_to_fp8x8(nk, a.inv_k_scale);
              vv[j] = f16x8_to_fp8x8(nv, a.inv_v_scale);
            }
          }
        }
      }
    };
    // scores, softmax state and P.V of one loaded batch
    auto consume = [&](int base, const Raw (&kk)[NJ], const Raw (&vv)[NJ]) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float s[NJ];
        float bm = -INFINITY;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float d = group_sum<LPR>(dot8(qv[gi], widen(kk[j])));
          const int tok = base + j * RPI + r;
          s[j] = tok < t1 ? d * sl2 : -INFINITY;
          bm = fmaxf(bm, s[j]);
        }
        // the reference moves (and the state is rescaled) only when a
        // batch max exceeds it by more than kSlack
        mt[gi] = fmaxf(mt[gi], bm);
        if (__builtin_amdgcn_ballot_w64(bm > m[gi] + kSlack)) {
          const float mn = fmaxf(m[gi], mt[gi]);
          const float al = fast_exp2(m[gi] - (mn == -INFINITY ? 0.f : mn));
          l[gi] *= al;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[gi][e] *= al;
          m[gi] = mn;
        }
        const float sh = m[gi] == -INFINITY ? 0.f : m[gi];
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          s[j] = fast_exp2(s[j] - sh);
          ps += s[j];
        }
        l[gi] += ps;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = acc[gi][e];
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            x = __builtin_fmaf(s[j], half_at(widen(vv[j]), e), x);
          acc[gi][e] = x;
        }
      }
    };
    for (int base = t0 + wave * TB; base < t1; base += W * TB) {
      Raw kk[NJ], vv[NJ];
      issue(base, kk, vv);
      consume(base, kk, vv);
    }
    // state relative to the true running max from here on (and in V's
    // units for an fp8 pool)
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float f = mt[gi] == -INFINITY ? 1.f : fast_exp2(m[gi] - mt[gi]);
      l[gi] *= f;
      const float fv = EB == 1 ? f * a.v_scale : f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gi][e] *= fv;
      m[gi] = mt[gi];
    }

    // merge the row groups of the wave (lanes sharing channel chunk c)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float mo = __shfl_xor(m[gi], off);
        const float lo = __shfl_xor(l[gi], off);
        const float mn = fmaxf(m[gi], mo);
        const float sh = mn == -INFINITY ? 0.f : mn;
        const float fa = fast_exp2(m[gi] - sh);
        const float fb = fast_exp2(mo - sh);
        l[gi] = l[gi] * fa + lo * fb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ao = __shfl_xor(acc[gi][e], off);
          acc[gi][e] = acc[gi][e] * fa + ao * fb;
        }
        m[gi] = mn;
      }
    }
    if (r == 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.acc[wave][gi][c * 8 + e] = acc[gi][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        sm.m[wave][gi] = m[gi];
        sm.l[wave][gi] = l[gi];
      }
    }
    merge_waves<D, G>(sm, sink);
  }
};

// ---------------------------------------------------------------------------
// Matrix-core range bodies
// ---------------------------------------------------------------------------
//
// MfmaSplitPath: the range body on the matrix cores (groups of g = 8, and 4
// at head size 128; multi-token and shared-prefix columns).  Two MFMA
// shapes, lane l holding A[l%16][k], B[k][l%16] for k in its group l/16's
// slice of K, and D[4(l/16)+i][l%16]:
//   S^T (16 rows x 16 columns) = K x Q^T with the 16x16x32 fp16 MFMA (A: 8
//        channels of a row per lane, B: the query channels of a column);
//   O^T (16 channels x 16 columns) += V^T x P^T with the 16x16x16 fp16
//        MFMA; P^T needs no data movement (the four scores a lane holds are
//        its B slots), V^T goes through LDS: token-major rows stored with
//        8-byte writes, and each lane's column (4 tokens of one channel)
//        taken with one transposing read (gfx950's ds_read_b64_tr_b16:
//        within a 16-lane group, lane j receives element j % 4 of the
//        8-byte rows that lanes 4e + j / 4 address; measured on MI355X 1-2%
//        faster than four 2-byte reads on GQA-4 and long-context decode).
// With one token per MFMA row a load instruction would fetch 64 bytes of
// each of 16 rows (half lines).  Here MFMA row i is token i/R and channel
// split i%R of each line chunk (R = 16/g), so one instruction fetches g
// tokens x R*64 contiguous bytes.  For the product to
// stay a matrix product, the split also indexes the columns: the 16 B
// columns are (head n%g, split n/g).  Column (h, q) multiplies every row by
// head h's channels of split q; only the rows of split q are kept, and the R
// lanes n, n+g, .. of a head add their splits into the full score (all with
// the same bits).  The extra columns then duplicate head h through softmax
// and P.V, and only columns < g are stored.  A tile of 16 tokens takes R
// MFMA row groups of g tokens; a lane's four score slots are tokens
// T(j) = (j/U)*g + (lane/16)*U + j%U of the tile (U = 4/R), and the P.V
// k-order follows T, which only changes which LDS rows V^T reads.  Every
// per-column quantity (running max, sum, rescale factor) lives in the lanes
// owning that column, and O^T's rows are channels, so the rescale is
// lane-local.
// CPL channels per lane per load: min(16 bytes, D/(4R) channels), >= 8.
//
// Full (F = true): all 16 columns distinct, for query columns of several
// tokens (multi-token rows).  The split still indexes the score product's
// columns, so the scores take R MFMA passes, pass k with B column n = query
// column k*G + n%G on split n/G; after the R-lane sum, lane column n keeps
// pass n/G, i.e. the score of its own column n.  Softmax and P.V then run
// once for 16 distinct columns: the loads stay whole-line and only the
// score product is repeated.
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, int B, int G, int EB, bool F = false, int W = kWaves>
struct MfmaSplitPath {
  static constexpr int kWavesWG = W;      // waves per workgroup
  static constexpr int R = 16 / G;              // channel splits = rows per token
  static constexpr int U = 4 / R;               // useful D values per lane per MFMA
  // 16-token tiles per batch.  The 16-column form at D = 128 takes two
  // (twice the bytes in flight per wave, three waves per SIMD): measured on
  // MI355X 4% faster on speculative verify (g = 4, 4 query tokens), while
  // the decode bodies keep one and four waves (32 tokens lose 3% on GQA-4).
  static constexpr int MT = (D == 128 && !F) ? 1 : 2;
  static constexpr int TB = 16 * MT;
  static constexpr int CPL = (16 / EB) < D / (4 * R) ? (16 / EB) : D / (4 * R);
  static constexpr int LC = R * 4 * CPL;        // channels of one line chunk
  static constexpr int KL = D / LC;             // loads per row group
  static constexpr int KS = CPL / 8;            // MFMA k-steps per load
  static constexpr int DT = D / 16;
  // Padded LDS row (halves), chosen for 2-byte V^T reads: the 4 lane
  // groups took rows U apart, 8 dwords each, and a row of VS/2 dwords with
  // U*VS/2 = 8 (mod 64) put the groups on disjoint banks (D + 4 left g = 4
  // four-way and g = 8 two-way conflicted); kept for the transposing reads.
  static constexpr int VS = D + (G == 4 ? 16 : 8);
  static_assert((U * VS / 2) % 64 == 8, "row padding of the V staging");
  static constexpr int kMinWaves = (D == 128 && F) ? 3 : 4;  // 168 / 128 VGPRs
  static constexpr int kColsMinWaves = kMinWaves;
  static constexpr int NS = F ? R : 1;          // score passes
  static constexpr int NCOL = F ? 16 : G;       // distinct columns
  static_assert(G == 8 || G == 4, "16 columns = g heads x R splits");
  static_assert(!F || EB == 2, "full columns: multi-token rows of an fp16 pool");
  static_assert(B % 16 == 0, "a tile must not straddle two blocks");
  static_assert(CPL >= 8 && CPL % 8 == 0 && KL * LC == D, "line chunks cover the row");
  using Raw = std::conditional_t<CPL * EB == 16, u32x4, u32x2>;

  struct SmemSplit {
    _Float16 vs[W][TB][VS];
    float acc[W][G][D];
    float m[W][G];
    float l[W][G];
  };
  // 16 columns: the V staging rows are dead once every wave has left its
  // loop, so the per-wave results take their place (4-wave workgroups:
  // four per CU)
  struct SmemFull {
    union {
      _Float16 vs[W][TB][VS];
      float acc[W][16][D];
    };
    float m[W][16];
    float l[W][16];
  };
  using Smem = std::conditional_t<F, SmemFull, SmemSplit>;

  __device__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (CPL * EB == 16) return load16(r, off);
    else return load8(r, off);
  }
  // fp16 channels s*8 .. s*8+7 of a loaded chunk
  __device__ static u32x4 part(const Raw& w, int s) {
    if constexpr (EB == 2) {
      return w;
    } else if constexpr (CPL == 8) {
      return fp8x8_to_f16x8(w);
    } else {
      const unsigned x = w.x, y = w.y, z = w.z, v = w.w;
      return s == 0 ? fp8x8_to_f16x8((u32x2){x, y}) : fp8x8_to_f16x8((u32x2){z, v});
    }
  }

  // this lane's chunk of the appended row (CPL channels from p) in the
  // pool's form: fp16 bits, or the codes the append stores
  __device__ static Raw appended(const _Float16* p, float inv) {
    if constexpr (EB == 2) {
      return *reinterpret_cast<const u32x4*>(p);
    } else if constexpr (CPL == 8) {
      return f16x8_to_fp8x8(*reinterpret_cast<const u32x4*>(p), inv);
    } else {
      const u32x2 lo = f16x8_to_fp8x8(*reinterpret_cast<const u32x4*>(p), inv);
      const u32x2 hi = f16x8_to_fp8x8(*reinterpret_cast<const u32x4*>(p + 8), inv);
      const unsigned a0 = lo.x, a1 = lo.y, b0 = hi.x, b1 = hi.y;
      return (u32x4){a0, a1, b0, b1};
    }
  }

  // t0 must be a multiple of 16; `last` as for ValuPath::run.
  // Column c (c < G) is query head kvh*G + c of sequence seq.
  template <class Sink>
  __device__ static void run(const DecodeArgs& a, Smem& sm, int kvh, int seq,
                             int t0, int t1, int last, Sink& sink) {
    static_assert(!F, "decode columns are the g heads");
    const int hd = (threadIdx.x & 15) % G;
    const int64_t qoff =
        ((int64_t)seq * a.num_heads + (int64_t)kvh * G + hd) * D;
    body<false>(a, sm, kvh, seq, t0, t1, last, sink, qoff, 0x7fffffff);
  }

  // The same over NCOL columns given by the caller (fp16 pools): the lanes
  // of column c = (lane%16)%NCOL pass the same query-row element offset qoff
  // (-1: an unused column, zero query) and key limit lim (keys t <= lim).
  template <class Sink>
  __device__ static void run_cols(const DecodeArgs& a, Smem& sm, int kvh,
                                  int seq, int t0, int t1, Sink& sink,
                                  int64_t qoff, int lim) {
    body<true>(a, sm, kvh, seq, t0, t1, -1, sink, qoff, lim);
  }

  template <bool kCols, class Sink>
  __device__ static void body(const DecodeArgs& a, Smem& sm, int kvh, int seq,
                              int t0, int t1, int last, Sink& sink,
                              int64_t qoff, int lim) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int q = col / G;                      // B column: split
    if (last >= 0) append_token<D, B, EB>(a, kvh, seq, last);

    // B operand of pass k, load kl, k-step s: the query row of column
    // k*G + col%G (F) or col%G, channels kl*LC + q*4*CPL + grp*CPL + s*8 ..
    f16x8 qb[NS][KL][KS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      int64_t qk = qoff;
      if constexpr (F) {       // as lane (grp, k*G + col%G) holds it
        const int src = (lane & 48) | (k * G + col % G);
        const uint64_t u = (uint64_t)qoff;
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)u, src);
        const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(u >> 32), src);
        qk = (int64_t)(((uint64_t)hi << 32) | lo);
      }
#pragma unroll
      for (int kl = 0; kl < KL; ++kl)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (!kCols || qk >= 0)
            v = *reinterpret_cast<const u32x4*>(
                a.query + qk + kl * LC + q * 4 * CPL + grp * CPL + s * 8);
          qb[k][kl][s] = __builtin_bit_cast(f16x8, v);
        }
    }

    BlockWindow bw;
    bw.init(a.block_tables + (size_t)seq * a.max_blocks_per_seq, t0 / B,
            (t1 + B - 1) / B, lane);
    const uint32_t row_stride = (uint32_t)a.num_kv_heads * D * EB;
    const uint64_t blk_bytes = (uint64_t)B * row_stride;
    const char* kbase = a.key_cache + (size_t)kvh * D * EB;
    const char* vbase = a.value_cache + (size_t)kvh * D * EB;
    const float sl2 = a.scale * kLog2e * (EB == 1 ? a.k_scale : 1.f);
    // A operand row of a row group: token col/R, channels (load kl)
    // kl*LC + (col%R)*4*CPL + grp*CPL ..
    const int rtok = col / R;
    const int rch = (col % R) * 4 * CPL + grp * CPL;

    float m = -INFINITY;                        // reference of column col % G
    float mt = -INFINITY;                       // its true running max
    float l = 0.f;                              // this lane's share of the sum
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    _Float16* vw = &sm.vs[wave][0][0];

    for (int base = t0 + wave * TB; base < t1; base += W * TB) {
      bw.cover(base / B, (base + TB - 1) / B, lane);
      Raw kr[MT][R][KL], vr[MT][R][KL];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int tile0 = base + mi * 16;       // wave-uniform
        const int lb = tile0 / B;
        const int blk = bw.block(lb);
        const __amdgpu_buffer_rsrc_t rk = block_rsrc<B>(
            kbase, blk, lb, t1, row_stride, blk_bytes, a.num_blocks);
        const __amdgpu_buffer_rsrc_t rv = block_rsrc<B>(
            vbase, blk, lb, t1, row_stride, blk_bytes, a.num_blocks);
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
          const uint32_t off =
              (uint32_t)(tile0 % B + rg * G + rtok) * row_stride + rch * EB;
#pragma unroll
          for (int kl = 0; kl < KL; ++kl) {
            kr[mi][rg][kl] = load(rk, off + kl * LC * EB);
            vr[mi][rg][kl] = load(rv, off + kl * LC * EB);
          }
        }
      }
      if (last >= 0 && base + TB > last) {   // the appended row
        const size_t src = ((size_t)seq * a.num_kv_heads + kvh) * D + rch;
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
          for (int rg = 0; rg < R; ++rg)
            if (base + mi * 16 + rg * G + rtok == last) {
#pragma unroll
              for (int kl = 0; kl < KL; ++kl) {
                kr[mi][rg][kl] = appended(a.new_key + src + kl * LC, a.inv_k_scale);
                vr[mi][rg][kl] = appended(a.new_value + src + kl * LC, a.inv_v_scale);
              }
            }
      }

      // scores of this lane's column (col % G; col under F): slot j =
      // token tile0 + T(j)
      float sc[MT][4];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
          float pv[U];
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kl = 0; kl < KL; ++kl)
#pragma unroll
              for (int s = 0; s < KS; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(f16x8, part(kr[mi][rg][kl], s)), qb[k][kl][s],
                    acc, 0, 0, 0);
            // rows 4grp + j: token (4grp + j)/R, split j%R; keep split q
            const float av[4] = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
            for (int u = 0; u < U; ++u) {
              float p = av[R * u];
#pragma unroll
              for (int j = 1; j < R; ++j) p = q == j ? av[j + R * u] : p;
              // sum over the R lanes of column col % G (bitwise equal in each)
              if constexpr (R >= 2) p += dpp<kRowRor8>(p);
              if constexpr (R >= 4) p += dpp<kRowRor4>(p);
              pv[u] = (NS == 1 || q == k) ? p : pv[u];
            }
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int tok = base + mi * 16 + rg * G + grp * U + u;
            sc[mi][rg * U + u] =
                (tok < t1 && (!kCols || tok <= lim)) ? pv[u] * sl2 : -INFINITY;
          }
        }
      }

      // V tile to LDS in token-major rows (8-byte stores)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int rg = 0; rg < R; ++rg)
#pragma unroll
          for (int kl = 0; kl < KL; ++kl)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              _Float16* dst =
                  vw + (mi * 16 + rg * G + rtok) * VS + kl * LC + rch + s * 8;
              const u32x4 v = part(vr[mi][rg][kl], s);
              reinterpret_cast<uint2*>(dst)[0] = make_uint2(v.x, v.y);
              reinterpret_cast<uint2*>(dst)[1] = make_uint2(v.z, v.w);
            }

      // online softmax for column col % G (max over the batch and the 4 groups)
      float bm = -INFINITY;
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) bm = fmaxf(bm, sc[mi][i]);
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      mt = fmaxf(mt, bm);
      if (__builtin_amdgcn_ballot_w64(bm > m + kSlack)) {
        const float mn = fmaxf(m, mt);
        const float al = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
        l *= al;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= al;
        m = mn;
      }
      const float sh = m == -INFINITY ? 0.f : m;
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[mi][i] = fast_exp2(sc[mi][i] - sh);
          l += sc[mi][i];
        }

      // O^T += V^T P^T, the tile's 16 tokens in the slot order T
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        f16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = (_Float16)sc[mi][i];
        // one transposing read per fragment: lane col of group grp
        // addresses channels dt*16 + 4*(col%4) .. +3 of slot 4*grp + col/4's
        // row and receives channel dt*16 + col of the group's four slots
        const int e = col / 4;
        const _Float16* vt0 =
            vw + (mi * 16 + grp * U + (e / U) * G + e % U) * VS + 4 * (col % 4);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f16x4 va = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vt0 + dt * 16)));
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb, o[dt], 0, 0, 0);
        }
      }
    }

    // state relative to the true max (and in V's units for an fp8 pool);
    // the sum over the 4 lane groups; then merge the waves through LDS
    {
      const float f = mt == -INFINITY ? 1.f : fast_exp2(m - mt);
      l *= f;
      const float fv = EB == 1 ? f * a.v_scale : f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= fv;
      m = mt;
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if constexpr (F) __syncthreads();   // acc overlays every wave's V rows
    if (col < NCOL) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.acc[wave][col][dt * 16 + grp * 4 + i] = o[dt][i];
      if (grp == 0) {
        sm.m[wave][col] = m;
        sm.l[wave][col] = l;
      }
    }
    merge_waves<D, NCOL>(sm, sink);
  }
};

// ---------------------------------------------------------------------------
// Fixed partitions (single pass and split-KV)
// ---------------------------------------------------------------------------

// Grid (kv heads, sequences, partitions): consecutive workgroup ids -- which
// the dispatcher deals round-robin to the 8 XCDs -- differ in kv head and
// sequence, so every XCD gets a share of each partition index; partition 0
// of every sequence is dispatched first, later (possibly empty) ones last.
template <class Path, int D, int B, int G>
__global__ __launch_bounds__(kThreads) void partition_kernel(DecodeArgs a) {
  __shared__ typename Path::Smem sm;
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const int p = blockIdx.z;
  const int H = a.num_heads;
  int n = a.context_lens[seq];
  const int max_tok = a.max_blocks_per_seq * B;
  n = n < max_tok ? n : max_tok;
  const int t0 = p * a.partition_size;
  // shared-prefix decode: partitions below part_start came from prefix_kernel
  if (a.split && a.part_start && p < a.part_start[seq]) return;
  if (n <= 0 || t0 >= n) {
    if (!a.split && p == 0) {
      for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
        a.out[((size_t)seq * H + (size_t)kvh * G) * D + idx] = (_Float16)0.f;
    }
    return;
  }
  const int t1 = (t0 + a.partition_size) < n ? (t0 + a.partition_size) : n;
  auto sink = [&](int gi, int d, float mx, float L, float O) {
    const size_t h = (size_t)kvh * G + gi;
    if (a.split) {
      const size_t pi = ((size_t)seq * H + h) * a.max_partitions + p;
      if (d == 0) {
        a.ws_max[pi] = mx * kLn2;
        a.ws_sum[pi] = L;
      }
      a.ws_out[pi * D + d] = O;
    } else {
      a.out[((size_t)seq * H + h) * D + d] = (_Float16)(O / L);
    }
  };
  const int last = (a.new_key && t1 == n) ? n - 1 : -1;
  Path::run(a, sm, kvh, seq, t0, t1, last, sink);
}

// Fold np partition states (m_p, s_p, O_p), rows base .. base+np-1 of the
// workspace, into one normalised fp16 output row with the §4.6 merge:
// M = max m_p, S = sum s_p e^(m_p - M), out = sum e^(m_p - M) O_p / S.
// NT threads; a row of O is read by D/2 lanes with 8-byte loads (one wave
// per row at D = 128), so the workgroup folds NT/(D/2) rows at once and each
// lane keeps several rows in flight: the fold is bound by the workspace
// read, not by one load's latency per partition.  Row slot r folds rows r,
// r + RPP, ...; the RPP partial sums are then added in slot order, so the
// result does not depend on timing.  Launches pick NT = 512 when rows may
// hold many partitions (long contexts) and 128 otherwise, where wider
// workgroups would mostly idle.
template <int NT>
constexpr int fold_rows_per_pass(int D) { return NT / (D / 2); }

template <int D, int NT>
__device__ __forceinline__ void fold_states(const ReduceArgs& a, size_t base,
                                            int np, _Float16* out_row) {
  constexpr int LPR = D / 2;                    // lanes per row
  constexpr int RPP = fold_rows_per_pass<NT>(D);
  constexpr int NW = NT / 64;
  __shared__ float wmax[NW];
  __shared__ float2 acc[RPP][LPR];
  __shared__ float sacc[RPP];
  const int t = threadIdx.x;
  float mx = -INFINITY;
  for (int p = t; p < np; p += NT) mx = fmaxf(mx, a.ws_max[base + p]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((t & 63) == 0) wmax[t >> 6] = mx;
  __syncthreads();
  mx = wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, wmax[w]);

  const int r = t / LPR, c = t % LPR;
  float sum = 0.f;
  float2 o = make_float2(0.f, 0.f);
#pragma unroll 4
  for (int p = r; p < np; p += RPP) {
    const float f = fast_exp2((a.ws_max[base + p] - mx) * kLog2e);
    sum += a.ws_sum[base + p] * f;
    const float2 v = reinterpret_cast<const float2*>(a.ws_out + (base + p) * D)[c];
    o.x += v.x * f;
    o.y += v.y * f;
  }
  acc[r][c] = o;
  if (c == 0) sacc[r] = sum;
  __syncthreads();
  if (t < LPR) {
    float S = 0.f, ox = 0.f, oy = 0.f;
#pragma unroll
    for (int q = 0; q < RPP; ++q) {
      S += sacc[q];
      ox += acc[q][t].x;
      oy += acc[q][t].y;
    }
    out_row[2 * t] = (_Float16)(ox / S);
    out_row[2 * t + 1] = (_Float16)(oy / S);
  }
}

// One workgroup per (query head, sequence): fold the sequence's non-empty
// fixed partitions.
template <int D, int NT>
__global__ __launch_bounds__(NT) void reduce_kernel(ReduceArgs a) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int H = a.num_heads;
  int n = a.context_lens[seq];
  n = n < a.max_tokens ? n : a.max_tokens;
  _Float16* o = a.out + ((size_t)seq * H + h) * D;
  if (n <= 0) {
    if (threadIdx.x < D) o[threadIdx.x] = (_Float16)0.f;
    return;
  }
  const int np = (n + a.partition_size - 1) / a.partition_size;
  fold_states<D, NT>(a, ((size_t)seq * H + h) * a.max_partitions, np, o);
}

// Columns of the whole-line body for query tokens or group members: VG =
// 4 distinct (row, head) columns at head size 128 for g <= 4, else 8 (the
// split body needs at least 8 channels per lane and load).
template <int D, int G>
constexpr int split_cols() {
  return (D == 128 && G <= 4) ? 4 : 8;
}

// ---------------------------------------------------------------------------
// Multi-token queries over the same tables (speculative verify, chunked
// prefill)
// ---------------------------------------------------------------------------
//
// Sequence i has T_i = cu_seqlens_q[i+1] - cu_seqlens_q[i] query tokens, the
// last T_i of its n_i cached tokens: query token j sits at position
// n_i - T_i + j and attends to keys t <= that position (causal within the
// chunk).  The matrix-core body runs with 16 columns = (query token, head)
// pairs: 16/g consecutive query tokens x the g heads of one kv head, so one
// workgroup reads each K/V byte of its key range once for all of them.
// Grid (kv heads, sequences x query tiles, partitions); every (query row,
// head, partition) state goes to the workspace and multi_reduce_kernel folds
// the partitions of each row.
template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    MfmaSplitPath<D, B, 8, 2, true>::kMinWaves))) void multi_kernel(DecodeArgs a) {
  using Path = MfmaSplitPath<D, B, 8, 2, true>;
  constexpr int QT = 16 / G;                   // query tokens per tile
  __shared__ typename Path::Smem sm;
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y / a.q_tiles;
  const int tile = blockIdx.y % a.q_tiles;
  const int p = blockIdx.z;
  const int H = a.num_heads;
  const int q0 = a.cu_seqlens_q[seq];
  const int T = a.cu_seqlens_q[seq + 1] - q0;
  const int max_tok = a.max_blocks_per_seq * B;
  int n = a.context_lens[seq];
  n = n < max_tok ? n : max_tok;
  const int j0 = tile * QT;
  if (T <= 0 || j0 >= T || n <= 0 || q0 < 0) return;
  int nq = T - j0 < QT ? T - j0 : QT;          // query tokens in this tile
  // rows past num_q_tokens (offsets that break the precondition) are skipped
  if (q0 + j0 + nq > a.num_q_tokens) nq = a.num_q_tokens - q0 - j0;
  if (nq <= 0) return;
  const int pos0 = n - T + j0;                 // position of its first token
  const int lim_max = pos0 + nq - 1;           // last key the tile reads
  const int t0 = p * a.partition_size;
  if (lim_max < 0 || t0 > lim_max) return;
  const int t1 = t0 + a.partition_size < lim_max + 1 ? t0 + a.partition_size
                                                     : lim_max + 1;
  const int col = threadIdx.x & 15;
  const int qj = col / G;
  const bool ok = qj < nq && pos0 + qj >= 0;
  const int64_t qoff =
      ok ? (((int64_t)q0 + j0 + qj) * H + (int64_t)kvh * G + col % G) * D : -1;
  auto sink = [&](int c, int d, float mx, float L, float O) {
    if (c / G >= nq) return;
    const size_t r = (size_t)q0 + j0 + c / G;
    const size_t pi = (r * H + (size_t)kvh * G + c % G) * a.max_partitions + p;
    if (d == 0) {
      a.ws_max[pi] = mx * kLn2;
      a.ws_sum[pi] = L;
    }
    a.ws_out[pi * D + d] = O;
  };
  Path::run_cols(a, sm, kvh, seq, t0, t1, sink, qoff, ok ? pos0 + qj : -1);
}

// ---------------------------------------------------------------------------
// Shared-prefix decode
// ---------------------------------------------------------------------------
//
// Sequences whose tables point at the same physical blocks for a prefix
// (parallel samples or a shared system prompt whose full blocks are shared
// by reference) form a group.  Each split-KV partition that lies inside the
// group's shared full blocks is computed once for all members: the
// matrix-core body runs with 16 columns = (member, head) pairs, 16/g members
// x the g heads of one kv head, reading the shared K/V once; each column
// keeps its member's context length as its key limit.  Every member's state
// goes to that member's own partition slot of the split-K workspace, where
// the partition kernel (which skips those partitions) and the reduce find
// it exactly as if it had been computed per sequence.

// Number of shared partitions a group gets (full partitions inside its
// shared full blocks, which count at most max_blocks_per_seq, and at most
// the launch's grid depth).
__device__ __forceinline__ int prefix_parts(const DecodeArgs& a, int g,
                                            int block_size) {
  int64_t blocks = a.grp_blocks[g];
  blocks = blocks < a.max_blocks_per_seq ? blocks : a.max_blocks_per_seq;
  const int64_t tok = blocks * block_size;
  int64_t parts = tok > 0 ? tok / a.partition_size : 0;
  return (int)(parts < a.grp_max_parts ? parts : a.grp_max_parts);
}

// part_start[s]: the shared partition count of the group that lists s (for
// the members the prefix kernel's tiles cover), else 0.  One workgroup:
// clear, then each thread takes member entries and finds their group by
// binary search over the offsets.  A sequence listed in several groups
// breaks a precondition (which group's partitions it receives is then
// unspecified).
__global__ __launch_bounds__(256) void prefix_marks_kernel(DecodeArgs a,
                                                           int* part_start,
                                                           int block_size) {
  for (int i = threadIdx.x; i < a.num_seqs; i += 256) part_start[i] = 0;
  __syncthreads();
  if (a.num_groups <= 0) return;
  const int total = a.grp_offsets[a.num_groups];
  for (int e = a.grp_offsets[0] + (int)threadIdx.x; e < total; e += 256) {
    int lo = 0, hi = a.num_groups - 1;      // last group with offset <= e
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.grp_offsets[mid] <= e) lo = mid; else hi = mid - 1;
    }
    if (e - a.grp_offsets[lo] >= a.grp_max_members) continue;
    const int s = a.grp_members[e];
    if (s >= 0 && s < a.num_seqs) part_start[s] = prefix_parts(a, lo, block_size);
  }
}

template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    MfmaSplitPath<D, B, 8, 2, true>::kMinWaves))) void prefix_kernel(DecodeArgs a) {
  using Path = MfmaSplitPath<D, B, 8, 2, true>;
  constexpr int MPT = 16 / G;                  // members per tile
  __shared__ typename Path::Smem sm;
  const int kvh = blockIdx.x;
  const int g = blockIdx.y / a.q_tiles;
  const int tile = blockIdx.y % a.q_tiles;
  const int p = blockIdx.z;
  const int H = a.num_heads;
  const int m0 = a.grp_offsets[g];
  const int cnt = a.grp_offsets[g + 1] - m0;
  const int j0 = tile * MPT;
  if (cnt <= 0 || j0 >= cnt || p >= prefix_parts(a, g, B)) return;
  const int nm = cnt - j0 < MPT ? cnt - j0 : MPT;
  const int lead = a.grp_members[m0];          // its row holds the shared blocks
  if (lead < 0 || lead >= a.num_seqs) return;
  const int max_tok = a.max_blocks_per_seq * B;
  const int t0 = p * a.partition_size;
  const int t1 = t0 + a.partition_size;
  const int col = threadIdx.x & 15;
  const int mj = col / G;
  const int ms = mj < nm ? a.grp_members[m0 + j0 + mj] : -1;
  int n = (ms >= 0 && ms < a.num_seqs) ? a.context_lens[ms] : 0;
  n = n < max_tok ? n : max_tok;
  const bool ok = n > t0;                      // member has keys here
  const int64_t qoff = ok ? ((int64_t)ms * H + (int64_t)kvh * G + col % G) * D : -1;
  auto sink = [&](int c, int d, float mx, float L, float O) {
    if (c / G >= nm) return;
    const int s = a.grp_members[m0 + j0 + c / G];
    if (s < 0 || s >= a.num_seqs) return;
    int ns = a.context_lens[s];
    ns = ns < max_tok ? ns : max_tok;
    if (ns <= t0) return;                      // the reduce never reads it
    const size_t pi =
        ((size_t)s * H + (size_t)kvh * G + c % G) * a.max_partitions + p;
    if (d == 0) {
      a.ws_max[pi] = mx * kLn2;
      a.ws_sum[pi] = L;
    }
    a.ws_out[pi * D + d] = O;
  };
  Path::run_cols(a, sm, kvh, lead, t0, t1, sink, qoff, ok ? n - 1 : -1);
}

// prefix_kernel on the whole-line body: VG/g members per tile.
template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) void prefix_split_kernel(DecodeArgs a) {
  constexpr int VG = split_cols<D, G>();
  using Path = MfmaSplitPath<D, B, VG, 2>;
  constexpr int MPT = VG / G;                  // members per tile
  __shared__ typename Path::Smem sm;
  const int kvh = blockIdx.x;
  const int g = blockIdx.y / a.q_tiles;
  const int tile = blockIdx.y % a.q_tiles;
  const int p = blockIdx.z;
  const int H = a.num_heads;
  const int m0 = a.grp_offsets[g];
  const int cnt = a.grp_offsets[g + 1] - m0;
  const int j0 = tile * MPT;
  if (cnt <= 0 || j0 >= cnt || p >= prefix_parts(a, g, B)) return;
  const int nm = cnt - j0 < MPT ? cnt - j0 : MPT;
  const int lead = a.grp_members[m0];          // its row holds the shared blocks
  if (lead < 0 || lead >= a.num_seqs) return;
  const int max_tok = a.max_blocks_per_seq * B;
  const int t0 = p * a.partition_size;
  const int t1 = t0 + a.partition_size;
  const int col = (threadIdx.x & 15) % VG;
  const int mj = col / G;
  const int ms = mj < nm ? a.grp_members[m0 + j0 + mj] : -1;
  int n = (ms >= 0 && ms < a.num_seqs) ? a.context_lens[ms] : 0;
  n = n < max_tok ? n : max_tok;
  const bool ok = n > t0;                      // member has keys here
  const int64_t qoff = ok ? ((int64_t)ms * H + (int64_t)kvh * G + col % G) * D : -1;
  auto sink = [&](int c, int d, float mx, float L, float O) {
    if (c / G >= nm) return;
    const int s = a.grp_members[m0 + j0 + c / G];
    if (s < 0 || s >= a.num_seqs) return;
    int ns = a.context_lens[s];
    ns = ns < max_tok ? ns : max_tok;
    if (ns <= t0) return;                      // the reduce never reads it
    const size_t pi =
        ((size_t)s * H + (size_t)kvh * G + c % G) * a.max_partitions + p;
    if (d == 0) {
      a.ws_max[pi] = mx * kLn2;
      a.ws_sum[pi] = L;
    }
    a.ws_out[pi * D + d] = O;
  };
  Path::run_cols(a, sm, kvh, lead, t0, t1, sink, qoff, ok ? n - 1 : -1);
}

// multi_kernel on the narrow form of the matrix-core body: VG/g query tokens
// per tile (used when that needs no more tiles than the 16-column form).
template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) void multi_split_kernel(DecodeArgs a) {
  constexpr int VG = split_cols<D, G>();
  using Path = MfmaSplitPath<D, B, VG, 2>;
  constexpr int QT = VG / G;                   // query tokens per tile
  __shared__ typename Path::Smem sm;
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y / a.q_tiles;
  const int tile = blockIdx.y % a.q_tiles;
  const int p = blockIdx.z;
  const int H = a.num_heads;
  const int q0 = a.cu_seqlens_q[seq];
  const int T = a.cu_seqlens_q[seq + 1] - q0;
  const int max_tok = a.max_blocks_per_seq * B;
  int n = a.context_lens[seq];
  n = n < max_tok ? n : max_tok;
  const int j0 = tile * QT;
  if (T <= 0 || j0 >= T || n <= 0 || q0 < 0) return;
  int nq = T - j0 < QT ? T - j0 : QT;
  if (q0 + j0 + nq > a.num_q_tokens) nq = a.num_q_tokens - q0 - j0;
  if (nq <= 0) return;
  const int pos0 = n - T + j0;
  const int lim_max = pos0 + nq - 1;
  const int t0 = p * a.partition_size;
  if (lim_max < 0 || t0 > lim_max) return;
  const int t1 = t0 + a.partition_size < lim_max + 1 ? t0 + a.partition_size
                                                     : lim_max + 1;
  const int cc = (threadIdx.x & 15) % VG;
  const int qj = cc / G;
  const bool ok = qj < nq && pos0 + qj >= 0;
  const int64_t qoff =
      ok ? (((int64_t)q0 + j0 + qj) * H + (int64_t)kvh * G + cc % G) * D : -1;
  auto sink = [&](int c, int d, float mx, float L, float O) {
    if (c / G >= nq) return;
    const size_t r = (size_t)q0 + j0 + c / G;
    const size_t pi = (r * H + (size_t)kvh * G + c % G) * a.max_partitions + p;
    if (d == 0) {
      a.ws_max[pi] = mx * kLn2;
      a.ws_sum[pi] = L;
    }
    a.ws_out[pi * D + d] = O;
  };
  Path::run_cols(a, sm, kvh, seq, t0, t1, sink, qoff, ok ? pos0 + qj : -1);
}

// One workgroup per (query head, query row): fold the partitions that hold
// the row's keys 0 .. pos (its causal limit).
template <int D, int NT>
__global__ __launch_bounds__(NT) void multi_reduce_kernel(ReduceArgs a) {
  const int h = blockIdx.x;
  const int r = blockIdx.y;
  const int H = a.num_heads;
  int lo = 0, hi = a.num_seqs - 1;              // sequence holding row r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_seqlens_q[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int T = a.cu_seqlens_q[lo + 1] - a.cu_seqlens_q[lo];
  int n = a.context_lens[lo];
  n = n < a.max_tokens ? n : a.max_tokens;
  const int pos = n - T + (r - a.cu_seqlens_q[lo]);
  _Float16* o = a.out + ((size_t)r * H + h) * D;
  if (n <= 0 || pos < 0) {
    if (threadIdx.x < D) o[threadIdx.x] = (_Float16)0.f;
    return;
  }
  int np = pos / a.partition_size + 1;
  np = np < a.max_partitions ? np : a.max_partitions;
  fold_states<D, NT>(a, ((size_t)r * H + h) * a.max_partitions, np, o);
}

// ---------------------------------------------------------------------------
// Balanced split
// ---------------------------------------------------------------------------
//
// Flat work order: sequence-major, then kv head, then column tile (one per
// pair except for wide multi-token chunks), then token; each unit spans
// a fixed pair cost (kPairCost, kFullPairCost for the 16-column multi-token
// form) and then its length padded to a multiple of 16 (span_len).  With T
// the flat total and C = ceil(T / grid) rounded up to 16, workgroup w owns
// flat positions [w*C, (w+1)*C).  Pairs of one
// sequence are adjacent, so neighbouring workgroups read neighbouring heads
// of the same token rows.
//
// The part of unit q = (seq*H_kv + kvh)*TL + tile (TL = the most tiles of
// any sequence, 1 for decode) inside workgroup w is one range.  A unit
// whose valid tokens [F, F+n) (F = the flat position of its token 0) fall
// in a single slice is finished in place.  Otherwise each of its k ranges
// stores its state in slot w + q (distinct: along the flat order w and q
// never decrease and one grows at every range boundary, so slots stay below
// grid + S*H_kv*TL), then counts itself in cnt[q].  The range that brings
// the count to k folds the k states with the online-softmax recurrence,
// writes the output and resets cnt[q] to zero for the next call.  Nothing
// waits on another workgroup.
// Partial states cross XCDs (each has its own L2), so they are stored and
// loaded with system-coherent accesses that bypass L2 (sc0 sc1) instead of
// fencing whole caches; a writer waits for its stores to be acknowledged
// before the range is counted with a system-scope atomic.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
}

// partial states a merging range loads before folding them
constexpr int kMergeBatch = 8;

__device__ __forceinline__ int64_t padded_len(int n, int max_tok) {
  n = n < max_tok ? n : max_tok;
  return n <= 0 ? 0 : (int64_t)((n + 15) & ~15);
}

// Flat span of one (sequence, kv head) pair: kPairCost units for the fixed
// cost of the range that starts it (table and query loads, the final merge),
// then its padded tokens; equal slices of this space then hold fewer tokens
// where they start more pairs.  Measured on MI355X with 8-wave workgroups
// (GQA-4 / Llama-2-13B, us): 32: 79.9 / 130.5, 64: 68.9 / 130.0, 96: 68.4 /
// 130.7, 128: 67.8 / 130.7 and 67.9 / 130.8 (64: 69.1 / 130.9 in the same
// run), 160: 69.5 / 132.0, 192: 68.1 / 132.6, 256: 69.6 / 133.8.  The
// 16-column multi-token form starts a pair at a higher cost (R query passes,
// a 16-column LDS accumulator, 16 rows to merge and store): 160 there takes
// 10% off the 4-token GQA-4 verify step (128: 4%, 192: 7%).
constexpr int kPairCost = 128;
constexpr int kFullPairCost = 160;
// The fp16 g = 4 matrix-core decode body charges 192: GQA-4 decode 66.2 ->
// 65.3 us (224: 66.0, 256: 66.1, 96: 67.5); the long-context g = 8 body and
// the vector body keep 128 (160 / 192: +0.2 / +0.3% and +0.7 / +0.6%).
template <class P>
struct DecodePairCost {
  static constexpr int value = kPairCost;
};
template <int B, int W>
struct DecodePairCost<MfmaSplitPath<128, B, 4, 2, false, W>> {
  static constexpr int value = 192;
};
template <int PC>
__device__ __forceinline__ int64_t span_len(int n, int max_tok) {
  const int64_t np = padded_len(n, max_tok);
  return np > 0 ? np + PC : 0;
}

__device__ __forceinline__ int64_t balanced_chunk(int64_t total, int grid) {
  const int64_t c = (total + grid - 1) / grid;
  return (c + 15) & ~(int64_t)15;
}

// Inclusive scan over the W waves of a workgroup: shuffles within each
// wave, then the wave totals through LDS.  `tot` receives the grand total.
template <int W>
__device__ __forceinline__ int64_t block_scan(int64_t v, int64_t* wave_sum,
                                              int64_t& tot) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_sum[w] = v;
  __syncthreads();
  int64_t before = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    before += i < w ? wave_sum[i] : 0;
    tot += wave_sum[i];
  }
  __syncthreads();
  return v + before;
}


// What a unit of the balanced split computes, and where its NC columns go.
// A unit is one column tile of a (sequence, kv head) pair.  DecodeCols: one
// tile, the sequence's query row x the pair's g heads.  MultiCols: the
// sequence's T query rows x g heads in tiles of NC/g rows, each row with its
// causal key limit, on the matrix-core body with NC = 4 or 8 columns (one
// tile, one score pass) or 16 (R score passes; ceil(T*g/16) tiles).
template <class P, int D, int G>
struct DecodeCols {
  using Path = P;
  static constexpr int NC = G;
  static constexpr int kMinWaves = P::kMinWaves;
  static constexpr int kPC = DecodePairCost<P>::value;   // flat units per pair
  // one column tile (the g heads) per (sequence, kv head)
  __device__ static int tiles(const DecodeArgs&, int) { return 1; }
  __device__ static int max_tiles(const DecodeArgs&) { return 1; }
  template <class Sink>
  __device__ static void run(const DecodeArgs& a, typename P::Smem& sm, int kvh,
                             int s, int, int n, int ta, int tv, int last,
                             Sink& sink) {
    P::run(a, sm, kvh, s, ta, tv, last, sink);
  }
  // output rows of a pair: computed once per range, then per column
  struct Out {
    int64_t base;
  };
  __device__ static Out out_of(const DecodeArgs& a, int s, int kvh, int) {
    return {((int64_t)s * a.num_heads + (int64_t)kvh * G) * D};
  }
  __device__ static int64_t out_elem(const DecodeArgs&, const Out& o, int c) {
    return o.base + (int64_t)c * D;
  }
  // every column of a decode range has keys, so L > 0
  __device__ static float finish(float O, float L) { return O / L; }
  __device__ static void clear_rows(const DecodeArgs& a, int s) {
    u32x4* o = reinterpret_cast<u32x4*>(a.out + (size_t)s * a.num_heads * D);
    for (int k = 0; k < a.num_heads * D / 8; ++k) o[k] = (u32x4){0u, 0u, 0u, 0u};
  }
};

template <class P, int NCOLS, int D, int G>
struct MultiCols {
  using Path = P;
  static constexpr int NC = NCOLS;
  static constexpr int kMinWaves = P::kColsMinWaves;
  static constexpr int kPC = NCOLS == 16 ? kFullPairCost : kPairCost;
  static constexpr int RT = NCOLS / G;         // query rows per column tile
  __device__ static int max_tiles(const DecodeArgs& a) {
    return a.q_tiles > 1 ? a.q_tiles : 1;
  }
  // column tiles of sequence s: its T rows, RT per tile (none without rows)
  // (at most max_tiles: rows past max_q_per_seq break a precondition and are
  // left alone rather than given another pair's counter)
  __device__ static int tiles(const DecodeArgs& a, int s) {
    const int T = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
    const int t = T > 0 ? (T + RT - 1) / RT : 0;
    return t < max_tiles(a) ? t : max_tiles(a);
  }
  // query row of column c of tile t (row t*RT + c/G of the sequence's
  // rows), -1 if none
  __device__ static int64_t row_of(const DecodeArgs& a, int s, int c, int t) {
    const int q0 = a.cu_seqlens_q[s];
    const int T = a.cu_seqlens_q[s + 1] - q0;
    const int qj = t * RT + c / G;
    if (q0 < 0 || qj >= T || q0 + qj >= a.num_q_tokens) return -1;
    return (int64_t)q0 + qj;
  }
  template <class Sink>
  __device__ static void run(const DecodeArgs& a, typename Path::Smem& sm, int kvh,
                             int s, int t, int n, int ta, int tv, int, Sink& sink) {
    const int col = (threadIdx.x & 15) % NC;
    const int64_t r = row_of(a, s, col, t);
    const int T = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
    const int pos = n - T + t * RT + col / G;  // this row's position
    const bool ok = r >= 0 && pos >= 0;
    const int64_t qoff =
        ok ? (r * a.num_heads + (int64_t)kvh * G + col % G) * D : -1;
    Path::run_cols(a, sm, kvh, s, ta, tv, sink, qoff, ok ? pos : -1);
  }
  struct Out {
    int s, kvh, t;
  };
  __device__ static Out out_of(const DecodeArgs&, int s, int kvh, int t) {
    return {s, kvh, t};
  }
  __device__ static int64_t out_elem(const DecodeArgs& a, const Out& o, int c) {
    const int64_t r = row_of(a, o.s, c, o.t);
    return r < 0 ? -1 : (r * a.num_heads + (int64_t)o.kvh * G + c % G) * D;
  }
  // a row placed before the first key (T > n) has none: zeros
  __device__ static float finish(float O, float L) { return L > 0.f ? O / L : 0.f; }
  __device__ static void clear_rows(const DecodeArgs& a, int s) {
    const int q0 = a.cu_seqlens_q[s];
    int q1 = a.cu_seqlens_q[s + 1];
    q1 = q1 < a.num_q_tokens ? q1 : a.num_q_tokens;
    for (int r = q0 < 0 ? 0 : q0; r < q1; ++r) {
      u32x4* o = reinterpret_cast<u32x4*>(a.out + (size_t)r * a.num_heads * D);
      for (int k = 0; k < a.num_heads * D / 8; ++k) o[k] = (u32x4){0u, 0u, 0u, 0u};
    }
  }
};

template <class Cols, int D, int B, int G>
__global__ __launch_bounds__(64 * Cols::Path::kWavesWG)
__attribute__((amdgpu_waves_per_eu(Cols::kMinWaves))) void balanced_kernel(
    DecodeArgs a) {
  constexpr int NC = Cols::NC;
  constexpr int NW = Cols::Path::kWavesWG;   // waves per workgroup
  constexpr int NT = 64 * NW;
  __shared__ typename Cols::Path::Smem sm;
  __shared__ int64_t wave_sum[NW];
  __shared__ int64_t found_start;
  __shared__ int found_seq;
  __shared__ int merge_here;
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int max_tok = a.max_blocks_per_seq * B;
  const int w = blockIdx.x;

  // Padded lengths, 256 sequences per pass: the total and the sequence whose
  // flat span holds this workgroup's first position (one pass if S <= 256).
  // The first workgroup also clears the outputs of empty sequences.
  if (threadIdx.x == 0) found_seq = -1;
  int64_t total_per_kvh = 0;
  int64_t my_len = 0, my_inc = 0;          // this thread's sequence (pass 0)
  for (int s0 = 0; s0 < S; s0 += NT) {
    const int si = s0 + (int)threadIdx.x;
    const int ns = si < S ? a.context_lens[si] : 1;
    const int64_t len = si < S ? span_len<Cols::kPC>(ns, max_tok) * Cols::tiles(a, si) : 0;
    if (w == 0 && ns <= 0) {
      if (a.slot_out) a.slot_out[si] = -1;
      Cols::clear_rows(a, si);
    }
    int64_t chunk = 0;
    const int64_t inc = block_scan<NW>(len, wave_sum, chunk);
    if (s0 == 0) {
      my_len = len;
      my_inc = inc;
    }
    total_per_kvh += chunk;
  }
  const int64_t total = total_per_kvh * Hkv;
  const int64_t C = balanced_chunk(total, gridDim.x);
  const int64_t start = (int64_t)w * C;
  if (total == 0 || start >= total) return;
  const int64_t end = start + C < total ? start + C : total;

  if (S <= NT) {
    // flat span of sequence si: [(inc - len) * H_kv, inc * H_kv)
    if (my_len > 0 && (my_inc - my_len) * Hkv <= start && start < my_inc * Hkv) {
      found_seq = (int)threadIdx.x;
      found_start = (my_inc - my_len) * Hkv;
    }
    __syncthreads();
  } else {
    int64_t run = 0;
    for (int s0 = 0; s0 < S; s0 += NT) {
      const int si = s0 + (int)threadIdx.x;
      const int64_t len =
          si < S ? span_len<Cols::kPC>(a.context_lens[si], max_tok) * Cols::tiles(a, si) * Hkv
                 : 0;
      int64_t chunk = 0;
      const int64_t inc = block_scan<NW>(len, wave_sum, chunk);
      if (len > 0 && run + inc - len <= start && start < run + inc) {
        found_seq = si;
        found_start = run + inc - len;
      }
      __syncthreads();
      if (found_seq >= 0) break;
      run += chunk;
    }
  }
  int s = found_seq;
  int64_t E = found_start;               // flat start of sequence s
  if (s < 0) return;                     // unreachable while start < total

  const int TL = Cols::max_tiles(a);
  int64_t pos = start;
  while (pos < end && s < S) {
    int n = a.context_lens[s];
    n = n < max_tok ? n : max_tok;
    const int64_t np = span_len<Cols::kPC>(n, max_tok);
    const int tl = Cols::tiles(a, s);
    if (np == 0 || tl == 0) {
      ++s;
      continue;
    }
    // the sequence's units: kv head-major, then column tile
    const int64_t u = (pos - E) / np;
    const int kvh = (int)(u / tl);
    const int tile = (int)(u % tl);
    const int64_t F = E + u * np + Cols::kPC;          // flat token 0
    const int64_t pair_end = E + (u + 1) * np;
    const int64_t seg_end = end < pair_end ? end : pair_end;
    const int ta = (int)(pos > F ? pos - F : 0);
    const int tb = (int)(seg_end > F ? seg_end - F : 0);
    const int tv = tb < n ? tb : n;
    if (ta < tv) {
      const int64_t w0 = F / C;
      const int64_t wl = (F + n - 1) / C;             // slice of the last token
      const int64_t q = ((int64_t)s * Hkv + kvh) * TL + tile;
      const int last = (a.new_key && tv == n) ? n - 1 : -1;
      const typename Cols::Out orow = Cols::out_of(a, s, kvh, tile);
      if (w0 == wl) {
        auto sink = [&](int gi, int d, float, float L, float O) {
          const int64_t oe = Cols::out_elem(a, orow, gi);
          if (oe >= 0) a.out[oe + d] = (_Float16)(Cols::finish(O, L));
        };
        Cols::run(a, sm, kvh, s, tile, n, ta, tv, last, sink);
      } else {
        const int64_t slot = (int64_t)w + q;
        auto sink = [&](int gi, int d, float mx, float L, float O) {
          const size_t pi = (size_t)slot * NC + gi;
          if (d == 0) {
            publish(a.ws_max + pi, mx * kLn2);
            publish(a.ws_sum + pi, L);
          }
          publish(a.ws_out + pi * D + d, O);
        };
        Cols::run(a, sm, kvh, s, tile, n, ta, tv, last, sink);
        // every thread's state stores acknowledged, then count this range
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
          merge_here = __hip_atomic_fetch_add(a.bal_count + q, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_SYSTEM) ==
                       (int)(wl - w0);
        __syncthreads();
        if (merge_here) {
          for (int idx = threadIdx.x; idx < NC * D; idx += NT) {
            const int gi = idx / D;
            const int d = idx % D;
            const int64_t oe = Cols::out_elem(a, orow, gi);
            if (oe < 0) continue;
            float mx = -INFINITY, L = 0.f, O = 0.f;
            // kMergeBatch ranges' states in flight at once, then folded
            for (int64_t w1 = w0; w1 <= wl; w1 += kMergeBatch) {
              float mp[kMergeBatch], lp[kMergeBatch], op[kMergeBatch];
#pragma unroll
              for (int k = 0; k < kMergeBatch; ++k) {
                const int64_t wr = w1 + k <= wl ? w1 + k : wl;
                const size_t pi = (size_t)(wr + q) * NC + gi;
                mp[k] = fetch(a.ws_max + pi);
                lp[k] = fetch(a.ws_sum + pi);
                op[k] = fetch(a.ws_out + pi * D + d);
              }
              float mn = mx;
#pragma unroll
              for (int k = 0; k < kMergeBatch; ++k) {
                if (w1 + k > wl) mp[k] = -INFINITY;      // past the last range
                mn = fmaxf(mn, mp[k]);
              }
              const float fa = fast_exp2((mx - mn) * kLog2e);   // 0 at first
              L *= fa;
              O *= fa;
#pragma unroll
              for (int k = 0; k < kMergeBatch; ++k) {
                const float fb = fast_exp2((mp[k] - mn) * kLog2e);
                L += lp[k] * fb;
                O += op[k] * fb;
              }
              mx = mn;
            }
            a.out[oe + d] = (_Float16)(Cols::finish(O, L));
          }
          if (threadIdx.x == 0) a.bal_count[q] = 0;    // ready for next call
        }
      }
    }
    pos = seg_end;
    if (pos == E + (int64_t)Hkv * tl * np) {
      E = pos;
      ++s;
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

// Bodies per group size, measured on MI355X.  Groups of 8, and of 4 at head
// size 128, run on the matrix cores with whole-line loads (g = 4 on c3: 4.4
// vs 3.9-4.0 TB/s for the vector body, fp8 48-50 vs 71-72 us; the earlier
// half-line matrix-core body had lost to the vector one).  The rest run the
// vector-ALU body with NJ loads in flight per wave batch: fp16 pools 8 for
// groups of 1-2, 2 for a group of 4 (fewer registers, four waves per SIMD);
// fp8 pools move half the bytes per load, so a group of 1 keeps 16 loads and
// a group of 4 keeps 4 in flight (+10% for g = 4); a group of 2 stays at 8
// (16 would halve its waves).
template <int G, int EB>
constexpr int valu_loads() {
  return EB == 2 ? (G >= 4 ? 2 : 8) : (G == 4 ? 4 : G == 2 ? 8 : 16);
}
// the decode columns run on the matrix cores (MfmaSplitPath below)
template <int D, int G>
constexpr bool is_mfma_decode() {
  return G == 8 || (D == 128 && G == 4);
}
template <int D, int B, int G, int EB = 2, int W = kWaves>
struct PathFor {
  using type = ValuPath<D, B, G, valu_loads<G, EB>(), EB, W>;
};
template <int D, int B, int EB, int W>
struct PathFor<D, B, 8, EB, W> {
  using type = MfmaSplitPath<D, B, 8, EB, false, W>;
};
template <int B, int EB, int W>
struct PathFor<128, B, 4, EB, W> {
  using type = MfmaSplitPath<128, B, 4, EB, false, W>;
};

// Waves per workgroup of the balanced decode kernel: 8 (two workgroups per
// CU) halves the slices' count against 4 waves and four workgroups, so
// fewer pairs are cut and merged.  Measured on MI355X: Llama-2-13B decode
// 135.6 -> 129.8 us, GQA-4 70.7 -> 68.6, long context 434.8 -> 433.5; 16
// waves (one workgroup per CU) were slower (141.7, 82.8).  The multi-token
// bodies keep 4 (the 16-column form at 8 waves fits one workgroup per CU:
// 4-token GQA-4 verify 82.4 -> 106.9 us), and so do the fp8 bodies (fp8
// decode kernel at 8 waves: Llama-2-13B 79.6 -> 83.4 us, long context at
// block 64 280.2 -> 314.2).  The matrix-core decode bodies (g = 8, g = 4 at
// head size 128) run 4 waves at two workgroups per CU instead: the same
// slices and cut pairs, half the waves, each with a longer run of batches.
// Measured on MI355X: GQA-4 67.6 -> 66.4 us, long context 434.1 -> 425.2
// (the vector body for g = 1 lost 1%: 130.9 -> 132.2; four workgroups of
// four waves per CU: GQA-4 69.6 at three, 70.7 at four).
template <int D, int G, int EB>
constexpr int decode_waves() {
  return EB == 2 && !is_mfma_decode<D, G>() ? 8 : 4;
}
// Workgroups per CU of the balanced decode grid (0: as many as fit).  The
// fp8 matrix-core bodies fit four 4-wave workgroups per CU; fewer run
// faster.  Measured on MI355X, fp8 decode kernel at grid 1024 / 768 / 512:
// g = 8 long context 239.7 / 218.5 / 215.4 us (B32) and 282.2 / 280.9 /
// 259.0 (B64); g = 4 GQA-4 42.8 / 40.8 / 47.8; the fp8 vector body (g = 1)
// is fastest at four (80.4 / 81.0 / 85.1).
template <int D, int G, int EB>
constexpr int decode_per_cu() {
  if (!is_mfma_decode<D, G>()) return 0;
  if (EB == 2) return 2;
  return G == 8 ? 2 : 3;
}

enum class Op { kPartition, kBalanced, kOccupancy, kMulti, kPrefix, kMultiSplit,
                kPrefixSplit, kMultiBalancedFull, kMultiFullOccupancy,
                kMultiBalancedSplit, kMultiSplitOccupancy };

// EB: bytes per cached element (2: fp16 pool, 1: fp8 e4m3 pool).  The fp8
// pool has the balanced kernel only.
template <int D, int B, int G, int EB>
static hipError_t run_op(Op op, const DecodeArgs* a, dim3 grid,
                         hipStream_t st, int* occ) {
  using P = typename PathFor<D, B, G, EB>::type;
  constexpr int DW = decode_waves<D, G, EB>();
  using DC = DecodeCols<typename PathFor<D, B, G, EB, DW>::type, D, G>;
  switch (op) {
    case Op::kBalanced:
      hipLaunchKernelGGL((balanced_kernel<DC, D, B, G>), grid, dim3(64 * DW), 0, st, *a);
      return hipGetLastError();
    case Op::kOccupancy: {
      const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          occ, reinterpret_cast<const void*>(&balanced_kernel<DC, D, B, G>), 64 * DW, 0);
      constexpr int cap = decode_per_cu<D, G, EB>();
      if (e == hipSuccess && cap > 0 && *occ > cap) *occ = cap;
      return e;
    }
    default:
      break;
  }
  if constexpr (EB == 2) {
    constexpr int VG = split_cols<D, G>();
    using MCS = MultiCols<MfmaSplitPath<D, B, VG, 2>, VG, D, G>;
    using MCF = MultiCols<MfmaSplitPath<D, B, 8, 2, true>, 16, D, G>;
    switch (op) {
      case Op::kPartition:
        hipLaunchKernelGGL((partition_kernel<P, D, B, G>), grid, dim3(kThreads), 0, st, *a);
        return hipGetLastError();
      case Op::kMulti:
        hipLaunchKernelGGL((multi_kernel<D, B, G>), grid, dim3(kThreads), 0, st, *a);
        return hipGetLastError();
      case Op::kPrefix:
        hipLaunchKernelGGL((prefix_kernel<D, B, G>), grid, dim3(kThreads), 0, st, *a);
        return hipGetLastError();
      case Op::kMultiSplit:
        hipLaunchKernelGGL((multi_split_kernel<D, B, G>), grid, dim3(kThreads), 0, st, *a);
        return hipGetLastError();
      case Op::kPrefixSplit:
        hipLaunchKernelGGL((prefix_split_kernel<D, B, G>), grid, dim3(kThreads), 0, st, *a);
        return hipGetLastError();
      case Op::kMultiBalancedFull:
        hipLaunchKernelGGL((balanced_kernel<MCF, D, B, G>), grid, dim3(kThreads), 0,
                           st, *a);
        return hipGetLastError();
      case Op::kMultiFullOccupancy:
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
            occ, reinterpret_cast<const void*>(&balanced_kernel<MCF, D, B, G>),
            kThreads, 0);
      case Op::kMultiBalancedSplit:
        hipLaunchKernelGGL((balanced_kernel<MCS, D, B, G>), grid, dim3(kThreads), 0,
                           st, *a);
        return hipGetLastError();
      case Op::kMultiSplitOccupancy:
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
            occ, reinterpret_cast<const void*>(&balanced_kernel<MCS, D, B, G>),
            kThreads, 0);
      default:
        break;
    }
  }
  return hipErrorInvalidValue;
}

template <int D, int B, int EB>
static hipError_t dispatch_db(Op op, int G, const DecodeArgs* a, dim3 grid,
                              hipStream_t st, int* occ) {
  switch (G) {
    case 1: return run_op<D, B, 1, EB>(op, a, grid, st, occ);
    case 2: return run_op<D, B, 2, EB>(op, a, grid, st, occ);
    case 4: return run_op<D, B, 4, EB>(op, a, grid, st, occ);
    case 8: return run_op<D, B, 8, EB>(op, a, grid, st, occ);
  }
  return hipErrorInvalidValue;
}

template <int D, int EB>
static hipError_t dispatch_d(Op op, int B, int G, const DecodeArgs* a, dim3 grid,
                             hipStream_t st, int* occ) {
  switch (B) {
    case 16: return dispatch_db<D, 16, EB>(op, G, a, grid, st, occ);
    case 32: return dispatch_db<D, 32, EB>(op, G, a, grid, st, occ);
    case 64: return dispatch_db<D, 64, EB>(op, G, a, grid, st, occ);
  }
  return hipErrorInvalidValue;
}

template <int EB>
static hipError_t dispatch_eb(Op op, int D, int B, int G, const DecodeArgs* a,
                              dim3 grid, hipStream_t st, int* occ) {
  switch (D) {
    case 64: return dispatch_d<64, EB>(op, B, G, a, grid, st, occ);
    case 128: return dispatch_d<128, EB>(op, B, G, a, grid, st, occ);
  }
  return hipErrorInvalidValue;
}

static hipError_t dispatch(Op op, int D, int B, int G, const DecodeArgs* a,
                           dim3 grid, hipStream_t st, int* occ, int eb = 2) {
  if (eb == 1) return dispatch_eb<1>(op, D, B, G, a, grid, st, occ);
  if (eb == 2) return dispatch_eb<2>(op, D, B, G, a, grid, st, occ);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int head_size, int block_size,
                         int group, dim3 grid, hipStream_t stream) {
  return dispatch(Op::kPartition, head_size, block_size, group, &a, grid,
                  stream, nullptr);
}

hipError_t launch_balanced(const DecodeArgs& a, int head_size, int block_size,
                           int group, int grid, hipStream_t stream, int elem_bytes) {
  return dispatch(Op::kBalanced, head_size, block_size, group, &a,
                  dim3(grid), stream, nullptr, elem_bytes);
}

int balanced_grid(int head_size, int block_size, int group, int elem_bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
      hipSuccess)
    return 0;
  int per_cu = 0;
  if (dispatch(Op::kOccupancy, head_size, block_size, group, nullptr, dim3(1),
               nullptr, &per_cu, elem_bytes) != hipSuccess)
    return 0;
  return per_cu > 0 ? per_cu * cus : 0;
}

hipError_t launch_multi(const DecodeArgs& a, int head_size, int block_size,
                        int group, dim3 grid, bool whole_line,
                        hipStream_t stream) {
  return dispatch(whole_line ? Op::kMultiSplit : Op::kMulti, head_size,
                  block_size, group, &a, grid, stream, nullptr);
}

hipError_t launch_prefix(const DecodeArgs& a, int head_size, int block_size,
                         int group, dim3 grid, bool whole_line,
                         hipStream_t stream) {
  return dispatch(whole_line ? Op::kPrefixSplit : Op::kPrefix, head_size,
                  block_size, group, &a, grid, stream, nullptr);
}

int split_columns(int head_size, int group) {
  return (head_size == 128 && group <= 4) ? 4 : 8;
}

hipError_t launch_prefix_marks(const DecodeArgs& a, int block_size,
                               int* part_start, hipStream_t stream) {
  hipLaunchKernelGGL(prefix_marks_kernel, dim3(1), dim3(256), 0, stream, a,
                     part_start, block_size);
  return hipGetLastError();
}

hipError_t launch_multi_balanced(const DecodeArgs& a, int head_size,
                                 int block_size, int group, int grid,
                                 bool whole_line, hipStream_t stream) {
  return dispatch(whole_line ? Op::kMultiBalancedSplit : Op::kMultiBalancedFull,
                  head_size, block_size, group, &a, dim3(grid), stream, nullptr);
}

int multi_balanced_grid(int head_size, int block_size, int group,
                        bool whole_line) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
      hipSuccess)
    return 0;
  int per_cu = 0;
  if (dispatch(whole_line ? Op::kMultiSplitOccupancy : Op::kMultiFullOccupancy,
               head_size, block_size, group, nullptr, dim3(1), nullptr,
               &per_cu) != hipSuccess)
    return 0;
  return per_cu > 0 ? per_cu * cus : 0;
}

// the partition folds: kMulti picks the per-query-row form
template <bool kMulti, int D, int NT>
static void fold_launch(const ReduceArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (kMulti)
    hipLaunchKernelGGL((multi_reduce_kernel<D, NT>), grid, dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL((reduce_kernel<D, NT>), grid, dim3(NT), 0, stream, a);
}

template <bool kMulti>
static hipError_t launch_fold(const ReduceArgs& a, int head_size, dim3 grid,
                              hipStream_t stream) {
  const bool wide = a.max_partitions >= 32;
  switch (head_size) {
    case 64:
      if (wide) fold_launch<kMulti, 64, 512>(a, grid, stream);
      else fold_launch<kMulti, 64, 128>(a, grid, stream);
      return hipGetLastError();
    case 128:
      if (wide) fold_launch<kMulti, 128, 512>(a, grid, stream);
      else fold_launch<kMulti, 128, 128>(a, grid, stream);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_multi_reduce(const ReduceArgs& a, int head_size,
                               int num_q_tokens, hipStream_t stream) {
  return launch_fold<true>(a, head_size, dim3(a.num_heads, num_q_tokens), stream);
}

hipError_t launch_reduce(const ReduceArgs& a, int head_size, int num_seqs,
                         hipStream_t stream) {
  return launch_fold<false>(a, head_size, dim3(a.num_heads, num_seqs), stream);
}

}  // namespace pa
