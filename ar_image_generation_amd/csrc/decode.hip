// sparse_decode_attn: split-KV decode attention over listed (kept) keys.
//
// Grid: one 256-thread workgroup per (query, kv head, chunk of `split`
// listed keys).  Each K/V row (head_dim elements, 128-512 bytes) is read by
// LPR = row_bytes / 16 consecutive lanes with one 16-byte load each, so a
// wave instruction moves 64 x 16 = 1 KiB and rows of a run are contiguous
// in memory.  A thread owns NP row slots of the chunk and issues all of its
// K and V loads before any arithmetic, so the whole chunk (up to 128 KiB per
// workgroup) is in flight at once: the kernel is bound by HBM bandwidth on
// the kept bytes and has no other use for the data, so it is not staged
// through LDS; LDS only carries the cross-wave softmax/output reduction.
//
// All hq/hkv query heads that share a kv head are served by the same
// workgroup, so each kept row is read once.  Scores are q . k scaled by
// log2(e)/sqrt(d) (folded into q) and reduced across a row's lanes with DPP;
// the chunk's max, sum and sum p*v follow.  A query whose list fits one
// chunk writes its normalised output directly; otherwise chunks leave
// (max, sum, unnormalised o) partials and merge_kernel combines them.
#include "common.h"

namespace da {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t page_stride, head_stride, slot_stride;
  const int32_t* block_table;
  int bt_stride, ps_shift, ps_mask;
  const int32_t* seq;
  const int32_t* count;
  const int32_t* idx;
  int n_q, hq, hkv, cap, split, max_split;
  float qscale;           // scale * log2(e)
  void* out;
  float* lse;
  float* ws_o;            // [n_q][hq][max_split][HD]
  float* ws_ml;           // [n_q][hq][max_split][2]
};

template <bool BF16>
__device__ inline void store_chunk(void* base, int64_t off, const float* x, int epl) {
  if constexpr (BF16) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = f32_to_bf16(x[2 * e]) | (f32_to_bf16(x[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + off) = u32x4{w[0], w[1], w[2], w[3]};
  } else {
    *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(base) + off) =
        u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  }
}

template <bool BF16, int HD, int GRP, int TMAX>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ES;            // elements per 16-byte chunk
  constexpr int LPR = HD * ES / 16;       // lanes per row
  constexpr int RPP = 256 / LPR;          // rows per pass of the workgroup
  constexpr int NP = (TMAX + RPP - 1) / RPP;
  constexpr int WROWS = 64 / LPR;         // row slots per wave per pass

  __shared__ float red_m[4][GRP];
  __shared__ float red_l[4][GRP];
  __shared__ float red_o[4][GRP][HD];

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int c = t % LPR;
  const int rsub = t / LPR;

  const int bid = blockIdx.x;
  const int s = bid % a.max_split;
  const int qg = bid / a.max_split;
  const int qi = qg / a.hkv;
  const int g = qg % a.hkv;

  int cnt = a.count[qi];
  cnt = cnt < a.cap ? cnt : a.cap;
  const int r0 = s * a.split;
  if (r0 >= cnt) return;
  const int nrows = cnt - r0 < a.split ? cnt - r0 : a.split;
  const int sq = a.seq[qi];

  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const int32_t* myidx = a.idx + (int64_t)qi * a.cap + r0;

  // ---- issue every K and V load of this thread's row slots
  u32x4 kr[NP], vr[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = p * RPP + rsub;
    if (r < nrows) {
      const int j = myidx[r];
      int64_t page, slot;
      if (a.block_table) {
        page = a.block_table[(int64_t)sq * a.bt_stride + (j >> a.ps_shift)];
        slot = j & a.ps_mask;
      } else {
        page = sq;
        slot = j;
      }
      const int64_t off = (page * a.page_stride + g * a.head_stride + slot * a.slot_stride + c * EPL) * ES;
      kr[p] = *reinterpret_cast<const u32x4*>(kb + off);
      vr[p] = *reinterpret_cast<const u32x4*>(vb + off);
    } else {
      kr[p] = u32x4{0, 0, 0, 0};
      vr[p] = u32x4{0, 0, 0, 0};
    }
  }

  // ---- this lane's slice of the GRP query heads, pre-scaled
  float qf[GRP][EPL];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const int64_t qoff = ((int64_t)qi * a.hq + g * GRP + h) * HD + c * EPL;
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.q) + qoff * ES);
    unpack<EPL>(w, qf[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] *= a.qscale;
  }

  // ---- scores (log2 domain)
  float sc[NP][GRP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float kx[EPL];
    unpack<EPL>(kr[p], kx);
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qf[h][e], kx[e], d);
      d = group_sum<LPR>(d);
      sc[p][h] = (p * RPP + rsub < nrows) ? d : -INFINITY;
    }
  }

  // ---- chunk max per head
  float mx[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    float m = sc[0][h];
#pragma unroll
    for (int p = 1; p < NP; ++p) m = fmaxf(m, sc[p][h]);
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    mx[h] = m;
  }
  if ((t & 63) == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) red_m[wave][h] = mx[h];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GRP; ++h)
    mx[h] = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));

  // ---- weights, their sum and sum p * v
  float ls[GRP];
  float acc[GRP][EPL];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float vx[EPL];
    unpack<EPL>(vr[p], vx);
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const float w = exp2f(sc[p][h] - mx[h]);   // 0 for empty slots
      ls[h] += w;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w, vx[e], acc[h][e]);
    }
  }
  // reduce over the row slots of the wave (lanes with the same chunk c)
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      ls[h] += __shfl_xor(ls[h], o);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
    }
  }
  // lanes 0..LPR-1 of each wave now hold the wave's totals
  if ((t & 63) < LPR) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[wave][h][c * EPL + e] = acc[h][e];
      if (c == 0) red_l[wave][h] = ls[h];
    }
  }
  __syncthreads();

  // ---- combine the four waves; one thread per (head, chunk)
  const bool single = cnt <= a.split;
  if (t < GRP * LPR) {
    const int h = t / LPR;
    const int cc = t % LPR;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      o[e] = red_o[0][h][cc * EPL + e] + red_o[1][h][cc * EPL + e] +
             red_o[2][h][cc * EPL + e] + red_o[3][h][cc * EPL + e];
    const float l = red_l[0][h] + red_l[1][h] + red_l[2][h] + red_l[3][h];
    const int head = g * GRP + h;
    const int64_t row = (int64_t)qi * a.hq + head;
    if (single) {
      const float inv = 1.f / l;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] *= inv;
      store_chunk<BF16>(a.out, row * HD + cc * EPL, o, EPL);
      if (a.lse && cc == 0) a.lse[row] = (mx[h] + log2f(l)) * kLn2;
    } else {
      float* dst = a.ws_o + (row * a.max_split + s) * HD + cc * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      if (cc == 0) {
        a.ws_ml[(row * a.max_split + s) * 2] = mx[h];
        a.ws_ml[(row * a.max_split + s) * 2 + 1] = l;
      }
    }
  }
}

// Log-sum-exp merge of a query head's chunk partials: one wave per
// (query, head); only queries whose list spans more than one chunk.
template <bool BF16, int HD>
__global__ void __launch_bounds__(64) merge_kernel(DecodeArgs a) {
  constexpr int EPT = HD / 64;
  const int row = blockIdx.x;           // query * hq + head
  const int qi = row / a.hq;
  const int lane = threadIdx.x;
  int cnt = a.count[qi];
  cnt = cnt < a.cap ? cnt : a.cap;
  if (cnt <= a.split) return;           // written directly by decode_kernel
  const int ns = (cnt + a.split - 1) / a.split;
  const float* ml = a.ws_ml + (int64_t)row * a.max_split * 2;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp2f(ml[2 * s] - M);
    L = fmaf(w, ml[2 * s + 1], L);
    const float* src = a.ws_o + ((int64_t)row * a.max_split + s) * HD;
#pragma unroll
    for (int e = 0; e < EPT; ++e) o[e] = fmaf(w, src[lane * EPT + e], o[e]);
  }
  const float inv = 1.f / L;
  if constexpr (BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + (int64_t)row * HD + lane * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) dst[e] = (uint16_t)f32_to_bf16(o[e] * inv);
  } else {
    float* dst = reinterpret_cast<float*>(a.out) + (int64_t)row * HD + lane * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) dst[e] = o[e] * inv;
  }
  if (a.lse && lane == 0) a.lse[row] = (M + log2f(L)) * kLn2;
}

typedef void (*decode_fn)(DecodeArgs);
typedef void (*merge_fn)(DecodeArgs);

template <bool BF16, int HD, int GRP>
static decode_fn pick_tmax(int split) {
  if (split <= 32) return decode_kernel<BF16, HD, GRP, 32>;
  if (split <= 64) return decode_kernel<BF16, HD, GRP, 64>;
  if (split <= 128) return decode_kernel<BF16, HD, GRP, 128>;
  return decode_kernel<BF16, HD, GRP, 256>;
}

template <bool BF16, int HD>
static decode_fn pick_grp(int grp, int split) {
  switch (grp) {
    case 1: return pick_tmax<BF16, HD, 1>(split);
    case 2: return pick_tmax<BF16, HD, 2>(split);
    case 4: return pick_tmax<BF16, HD, 4>(split);
    default: return pick_tmax<BF16, HD, 8>(split);
  }
}

static int64_t n_splits(int32_t cap, int32_t split) { return (int64_t(cap) + split - 1) / split; }

}  // namespace da

using namespace da;

extern "C" int64_t da_decode_workspace_bytes(int32_t n_q, int32_t hq, int32_t head_dim,
                                             int32_t cap, int32_t split) {
  if (n_q < 0 || hq < 1 || head_dim < 1 || cap < 1 || split < 1)
    return fail(DA_EINVAL, "workspace sizing: invalid sizes");
  const int64_t ns = n_splits(cap, split);
  if (ns <= 1) return 0;
  const int64_t rows = int64_t(n_q) * hq * ns;
  const int64_t o_bytes = ((rows * head_dim * 4) + 255) / 256 * 256;
  return o_bytes + rows * 2 * 4;
}

extern "C" int da_sparse_decode_attn(const void* q, da_dtype dtype, int32_t n_q, int32_t hq,
                                     int32_t hkv, int32_t head_dim, float scale,
                                     const da_kv_cache* kv, const int32_t* seq,
                                     const int32_t* count, const int32_t* idx, int32_t cap,
                                     int32_t split, void* out, float* lse, void* workspace,
                                     int64_t ws_bytes, void* stream) {
  if (n_q < 0) return fail(DA_EINVAL, "n_q=%d < 0", n_q);
  if (hq < 1 || hkv < 1 || hq % hkv) return fail(DA_EINVAL, "hq=%d hkv=%d: need hq %% hkv == 0", hq, hkv);
  if (!kv) return fail(DA_EINVAL, "kv descriptor is NULL");
  if (cap < 1 || split < 1) return fail(DA_EINVAL, "cap=%d split=%d must be >= 1", cap, split);
  if (dtype != DA_F32 && dtype != DA_BF16) return fail(DA_ENOTSUP, "dtype %d not supported", (int)dtype);
  if (head_dim != 64 && head_dim != 128) return fail(DA_ENOTSUP, "head_dim %d not in {64, 128}", head_dim);
  const int grp = hq / hkv;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(DA_ENOTSUP, "hq/hkv=%d not in {1, 2, 4, 8}", grp);
  if (split > 256) return fail(DA_ENOTSUP, "split=%d > 256", split);
  if (kv->block_table) {
    if (!is_pow2(kv->page_size)) return fail(DA_EINVAL, "page_size=%d not a power of two", kv->page_size);
    if (kv->bt_stride < 1) return fail(DA_EINVAL, "bt_stride=%d < 1", kv->bt_stride);
  }
  if (kv->page_stride < 0 || kv->head_stride < 0 || kv->slot_stride < 0)
    return fail(DA_EINVAL, "negative cache stride");
  if (n_q > 0 && (!q || !out || !seq || !count || !idx || !kv->k || !kv->v))
    return fail(DA_EINVAL, "q, out, seq, count, idx, kv->k and kv->v must be non-NULL");
  const int esz = dtype == DA_BF16 ? 2 : 4;
  if (((kv->page_stride | kv->head_stride | kv->slot_stride) * esz) % 16 ||
      ((uintptr_t)kv->k | (uintptr_t)kv->v | (uintptr_t)q | (uintptr_t)out) % 16)
    return fail(DA_EINVAL, "cache rows, q and out must be 16-byte aligned");
  const int64_t need = da_decode_workspace_bytes(n_q, hq, head_dim, cap, split);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(DA_ECAPACITY, "workspace %lld bytes < %lld needed", (long long)ws_bytes, (long long)need);
  if (need > 0 && (uintptr_t)workspace % 256) return fail(DA_EINVAL, "workspace not 256-byte aligned");
  clear_error();
  if (n_q == 0) return DA_OK;

  const int64_t ns = n_splits(cap, split);
  DecodeArgs a;
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.page_stride = kv->page_stride;
  a.head_stride = kv->head_stride;
  a.slot_stride = kv->slot_stride;
  a.block_table = kv->block_table;
  a.bt_stride = kv->bt_stride;
  a.ps_shift = kv->block_table ? ilog2(kv->page_size) : 0;
  a.ps_mask = kv->block_table ? kv->page_size - 1 : 0;
  a.seq = seq;
  a.count = count;
  a.idx = idx;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.cap = cap;
  a.split = split;
  a.max_split = (int)ns;
  a.qscale = scale * kLog2e;
  a.out = out;
  a.lse = lse;
  const int64_t rows = int64_t(n_q) * hq * ns;
  a.ws_o = need > 0 ? reinterpret_cast<float*>(workspace) : nullptr;
  a.ws_ml = need > 0 ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                                ((rows * head_dim * 4) + 255) / 256 * 256)
                     : nullptr;

  const int64_t blocks = int64_t(n_q) * hkv * ns;
  if (blocks > 0x7fffffff) return fail(DA_ENOTSUP, "grid of %lld workgroups too large", (long long)blocks);
  decode_fn dk;
  merge_fn mk;
  if (dtype == DA_BF16) {
    dk = head_dim == 64 ? pick_grp<true, 64>(grp, split) : pick_grp<true, 128>(grp, split);
    mk = head_dim == 64 ? merge_kernel<true, 64> : merge_kernel<true, 128>;
  } else {
    dk = head_dim == 64 ? pick_grp<false, 64>(grp, split) : pick_grp<false, 128>(grp, split);
    mk = head_dim == 64 ? merge_kernel<false, 64> : merge_kernel<false, 128>;
  }
  hipLaunchKernelGGL(dk, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  int rc = check_launch("decode_kernel");
  if (rc) return rc;
  if (ns > 1) {
    hipLaunchKernelGGL(mk, dim3((unsigned)(int64_t(n_q) * hq)), dim3(64), 0, (hipStream_t)stream, a);
    rc = check_launch("merge_kernel");
  }
  return rc;
}
