// Paged decode attention for gfx950 (CDNA4, wave64).
//
// What it computes: vLLM book ch.4 "PagedAttention：虚拟内存的启示", §4.5
// (walk the block table in logical order, read each physical block) and §4.6
// (online softmax; fp32 statistics and accumulators).
//
// Work decomposition.  One workgroup (4 waves) owns one (kv head, sequence,
// partition).  A partition is a run of whole blocks (P tokens, P a multiple of
// the block size); the single-pass entry point uses one partition per
// sequence.  The workgroup serves all g query heads of its kv head, so each
// K/V byte is fetched from HBM once and reused from registers g times.
//
// Inside a wave, a 16-byte load per lane covers one token row of one head
// (D/8 lanes per row), so one load instruction reads D*2*64/16 bytes of
// consecutive memory per row group -- whole 128-byte lines.  A wave walks a
// batch of TB tokens (NJ loads of K and NJ of V per lane in flight at once);
// the four waves take batches round-robin.  Physical block ids for the
// partition are fetched once with one vector load per wave (lane k holds
// logical block k of the current 64-block window) and broadcast with
// v_readlane, so the table read sits off the critical path of the K/V loads.
// Each block gets its own buffer resource whose record count ends at the
// last valid token: slots past context_len are never fetched, so padding may
// hold anything (Inf/NaN included) without reaching the result.
//
// Each row group (D/8 lanes = one token of a load) keeps its own online
// softmax state (m, l, acc[8] per head, replicated in the row).  The dot
// product is reduced across the row with four DPP adds (bitwise identical in
// every lane); everything else is lane-local until the end, where the row
// groups are merged with cross-lane shuffles, and the waves through LDS.
// Scores are kept in base-2 units (x * log2 e) so every exponential is a
// single v_exp_f32.
#include "common.h"
#include "decode.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, int B, int G, int NJ>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8;          // lanes per token row
  constexpr int RPI = 64 / LPR;       // token rows per wave load
  constexpr int TB = RPI * NJ;        // tokens per wave batch
  constexpr int NW = 4;               // waves per workgroup
  static_assert(B % RPI == 0, "a load must not straddle two blocks");

  __shared__ float sm_acc[NW][G][D];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];

  // grid (kv heads, sequences, partitions): consecutive workgroup ids -- which
  // the dispatcher deals round-robin to the 8 XCDs -- differ in kv head and
  // sequence, so every XCD gets a share of each partition index; partition 0
  // of every sequence is dispatched first, the (possibly empty) later
  // partitions last.
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const int p = blockIdx.z;
  const int H = a.num_heads;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;

  int n = a.context_lens[seq];
  const int max_tok = a.max_blocks_per_seq * B;
  n = n < max_tok ? n : max_tok;
  const int t0 = p * a.partition_size;
  if (n <= 0 || t0 >= n) {
    if (!a.split && p == 0) {
      for (int idx = threadIdx.x; idx < G * D; idx += 256)
        a.out[((size_t)seq * H + (size_t)kvh * G) * D + idx] = (_Float16)0.f;
    }
    return;
  }
  const int t1 = (t0 + a.partition_size) < n ? (t0 + a.partition_size) : n;

  // this lane's 8 channels of each query head of the group
  u32x4 qv[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
    qv[gi] = *reinterpret_cast<const u32x4*>(
        a.query + ((size_t)seq * H + (size_t)kvh * G + gi) * D + c * 8);

  const int* bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
  const int lb_end = (t1 + B - 1) / B;
  int win = t0 / B;                          // logical block held by lane 0
  int ids = (win + lane < lb_end) ? bt[win + lane] : 0;

  const uint32_t row_stride = (uint32_t)a.num_kv_heads * D * 2;
  const uint64_t blk_bytes = (uint64_t)B * row_stride;
  const char* kbase = a.key_cache + (size_t)kvh * D * 2;
  const char* vbase = a.value_cache + (size_t)kvh * D * 2;
  const float sl2 = a.scale * kLog2e;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = -INFINITY;
    l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
  }

  for (int base = t0 + wave * TB; base < t1; base += NW * TB) {
    // keep the id window over every block this batch touches
    if ((base + TB - 1) / B >= win + 64) {
      win = base / B;
      ids = (win + lane < lb_end) ? bt[win + lane] : 0;
    }
    u32x4 kk[NJ], vv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int tok0 = base + j * RPI;       // wave-uniform
      const int lb = tok0 / B;
      const int blk = __builtin_amdgcn_readlane(ids, lb - win);
      int valid = t1 - lb * B;
      valid = valid < B ? valid : B;
      const bool ok = valid > 0 && (unsigned)blk < (unsigned)a.num_blocks;
      const uint32_t bytes = ok ? (uint32_t)valid * row_stride : 0u;
      const uint64_t boff = ok ? (uint64_t)blk * blk_bytes : 0;
      const uint32_t off = (uint32_t)(tok0 % B + r) * row_stride + c * 16;
      kk[j] = load16(make_rsrc(kbase + boff, bytes), off);
      vv[j] = load16(make_rsrc(vbase + boff, bytes), off);
    }

#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float s[NJ];
      float bm = -INFINITY;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float d = group_sum<LPR>(dot8(qv[gi], kk[j]));
        const int tok = base + j * RPI + r;
        s[j] = tok < t1 ? d * sl2 : -INFINITY;
        bm = fmaxf(bm, s[j]);
      }
      const float mn = fmaxf(m[gi], bm);
      const float sh = mn == -INFINITY ? 0.f : mn;
      const float al = fast_exp2(m[gi] - sh);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        s[j] = fast_exp2(s[j] - sh);
        ps += s[j];
      }
      l[gi] = l[gi] * al + ps;
      m[gi] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[gi][e] * al;
#pragma unroll
        for (int j = 0; j < NJ; ++j) x = __builtin_fmaf(s[j], half_at(vv[j], e), x);
        acc[gi][e] = x;
      }
    }
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
      for (int e = 0; e < 8; ++e) sm_acc[wave][gi][c * 8 + e] = acc[gi][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      sm_m[wave][gi] = m[gi];
      sm_l[wave][gi] = l[gi];
    }
  }
  __syncthreads();

  // merge the waves; one thread per (head of the group, channel)
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int gi = idx / D;
    const int d = idx % D;
    float mx = sm_m[0][gi];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, sm_m[w][gi]);
    const float sh = mx == -INFINITY ? 0.f : mx;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm_m[w][gi] - sh);
      L += sm_l[w][gi] * f;
      O += sm_acc[w][gi][d] * f;
    }
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
  }
}

// One workgroup of D threads per (query head, sequence): fold the partition
// states in order with the online-softmax recurrence.
template <int D>
__global__ __launch_bounds__(D) void reduce_kernel(ReduceArgs a) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int d = threadIdx.x;
  const int H = a.num_heads;
  int n = a.context_lens[seq];
  n = n < a.max_tokens ? n : a.max_tokens;
  _Float16* o = a.out + ((size_t)seq * H + h) * D + d;
  if (n <= 0) {
    *o = (_Float16)0.f;
    return;
  }
  const int np = (n + a.partition_size - 1) / a.partition_size;
  const size_t base = ((size_t)seq * H + h) * a.max_partitions;
  float mx = -INFINITY;
  for (int p = 0; p < np; ++p) mx = fmaxf(mx, a.ws_max[base + p]);
  float S = 0.f, O = 0.f;
  for (int p = 0; p < np; ++p) {
    const float f = fast_exp2((a.ws_max[base + p] - mx) * kLog2e);
    S += a.ws_sum[base + p] * f;
    O += a.ws_out[(base + p) * D + d] * f;
  }
  *o = (_Float16)(O / S);
}

template <int D, int B, int G>
static hipError_t launch_dbg(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  constexpr int NJ = 8;
  hipLaunchKernelGGL((decode_partition_kernel<D, B, G, NJ>), grid, dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

template <int D, int B>
static hipError_t launch_db(const DecodeArgs& a, int G, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1: return launch_dbg<D, B, 1>(a, grid, st);
    case 2: return launch_dbg<D, B, 2>(a, grid, st);
    case 4: return launch_dbg<D, B, 4>(a, grid, st);
    case 8: return launch_dbg<D, B, 8>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, int B, int G, dim3 grid,
                           hipStream_t st) {
  switch (B) {
    case 16: return launch_db<D, 16>(a, G, grid, st);
    case 32: return launch_db<D, 32>(a, G, grid, st);
    case 64: return launch_db<D, 64>(a, G, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int head_size, int block_size,
                         int group, dim3 grid, hipStream_t stream) {
  switch (head_size) {
    case 64: return launch_d<64>(a, block_size, group, grid, stream);
    case 128: return launch_d<128>(a, block_size, group, grid, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, int head_size, int num_seqs,
                         hipStream_t stream) {
  dim3 grid(a.num_heads, num_seqs);
  switch (head_size) {
    case 64:
      hipLaunchKernelGGL(reduce_kernel<64>, grid, dim3(64), 0, stream, a);
      return hipGetLastError();
    case 128:
      hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(128), 0, stream, a);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
