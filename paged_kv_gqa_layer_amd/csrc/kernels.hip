// gfx950 (CDNA4) kernels for paged-KV grouped-query attention.
//
// What is computed ("nx_f32_attn_paged.nx source", header comment and
// nx_f32_attn_with_paged; "nx_f32_gqa_attention.nx source", header):
// query head h reads kv head h / group; query i of a row sits at position
// total_k - n_q + i and (causal) sees keys 0..that position; the output is
// softmax(q K^T * scale) V written at columns [h*head_dim, (h+1)*head_dim) of
// the query's output row.
//
// Every kernel is a template over the K/V address map (PagedMap: through the
// page table; ContigMap: a contiguous cache).  The arithmetic does not depend
// on the map, so the paged and contiguous forms are bit-identical.
//
// Scores are kept in base-2 units: q is prescaled by scale*log2(e) and the
// softmax uses exp2; the split merge uses the same units.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "device.hpp"

namespace pkv {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// DPP row (16-lane) permutations.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same
// bits (each stage adds a lane's value to its partner's, and IEEE addition
// commutes).  Pairings: xor 1, xor 2, mirror within 8 lanes, rotate by 8.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x128>(v);  // row_ror:8
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float4 ld4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

// Streaming load: K/V bytes a decode wave reads are used by that wave only,
// so they are fetched with the non-temporal hint (they are not kept in the
// caches for other workgroups).
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld4_stream(const float* p) {
  const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(r.x, r.y, r.z, r.w);
}
// Streaming store: the decode kernel's split partials are read once, by the
// merge launch; written with the non-temporal hint they do not take L2 lines
// from the K/V stream (the decode launch is 1% faster, the merge 2 us
// slower).  The verify kernel's partials stay ordinary stores: streaming
// them made it slower.
__device__ __forceinline__ void st4_stream(float* p, float4 v) {
  const f32x4 r = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ float dot8(const float4& ka, const float4& kb,
                                      const float (&qa)[4],
                                      const float (&qb)[4]) {
  float s = ka.x * qa[0];
  s = fmaf(ka.y, qa[1], s);
  s = fmaf(ka.z, qa[2], s);
  s = fmaf(ka.w, qa[3], s);
  s = fmaf(kb.x, qb[0], s);
  s = fmaf(kb.y, qb[1], s);
  s = fmaf(kb.z, qb[2], s);
  s = fmaf(kb.w, qb[3], s);
  return s;
}

// Rotary embedding, neox form ("nx_f32_llama_v4b.nx source",
// nx_f32_llama_block_forward_v4b, RoPE step): dims i and i + head_dim/2 of a
// head turn together by the angle of (position, i).  cs is the rotary table,
// [positions][head_dim/2] pairs (cos, sin) in double; the rotation runs in
// double and rounds once to float.
__device__ __forceinline__ void rotate_pair(float& lo, float& hi,
                                            const double2 cs) {
  const double a = lo, b = hi;
  lo = static_cast<float>(a * cs.x - b * cs.y);
  hi = static_cast<float>(a * cs.y + b * cs.x);
}

// ---------------------------------------------------------------------------
// Append: scatter new K/V rows to their (page, slot).  One thread per VEC
// floats; a row of one kv head is head_dim contiguous floats on both sides.
// With rotary embedding (ROPE), a thread takes VEC floats of the first half
// of a head and the VEC floats they pair with in the second half, and turns
// the K pairs by the row's position before storing them (V is stored as is).
// ---------------------------------------------------------------------------
// The scatter of rows [r][t] (element e of the flattened [rows][n][units]
// grid), from K / V into the pool.  ONE: one new row per sequence, written to
// the RowDesc's append_block (no page-table read).
template <int VEC, class Map, bool ROPE, bool ONE>
__device__ __forceinline__ void append_elems(
    const Map& m, const RowDesc* __restrict__ rows, const float* __restrict__ K,
    const float* __restrict__ V, int32_t n, int32_t kv_dim, int32_t head_dim,
    int64_t total, const double2* __restrict__ cs) {
  const int32_t span = ROPE ? head_dim / 2 : head_dim;  // floats per head unit
  const int32_t per_row = (ROPE ? kv_dim / 2 : kv_dim) / VEC;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rt = e / per_row;
    const int32_t c = static_cast<int32_t>(e - rt * per_row) * VEC;
    const int32_t r = static_cast<int32_t>(rt / n);
    const int32_t t = static_cast<int32_t>(rt - (int64_t)r * n);
    const RowDesc rd = rows[r];
    const int32_t pos = rd.start + t;
    const int32_t kvh = c / span;
    const int32_t d = c - kvh * span;
    float* pg;
    if constexpr (ONE) pg = m.block(rd.append_block, kvh);
    else pg = m.page(rd, pos / m.block_size, kvh);
    float* dst = pg + (int64_t)(pos % m.block_size) * head_dim + d;
    const int64_t src = rt * kv_dim + (int64_t)kvh * head_dim + d;
    if constexpr (ROPE) {
      const int32_t half = span;
      const double2* cr = cs + (int64_t)pos * half + d;
      float klo[VEC], khi[VEC], vlo[VEC], vhi[VEC];
      if constexpr (VEC == 4) {
        const float4 a = ld4(K + src), b = ld4(K + src + half);
        const float4 va = ld4(V + src), vb = ld4(V + src + half);
        klo[0] = a.x; klo[1] = a.y; klo[2] = a.z; klo[3] = a.w;
        khi[0] = b.x; khi[1] = b.y; khi[2] = b.z; khi[3] = b.w;
        vlo[0] = va.x; vlo[1] = va.y; vlo[2] = va.z; vlo[3] = va.w;
        vhi[0] = vb.x; vhi[1] = vb.y; vhi[2] = vb.z; vhi[3] = vb.w;
      } else {
        klo[0] = K[src];
        khi[0] = K[src + half];
        vlo[0] = V[src];
        vhi[0] = V[src + half];
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) rotate_pair(klo[j], khi[j], cr[j]);
      if constexpr (VEC == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(klo[0], klo[1], klo[2], klo[3]);
        *reinterpret_cast<float4*>(dst + half) = make_float4(khi[0], khi[1], khi[2], khi[3]);
        *reinterpret_cast<float4*>(dst + m.v_off) = make_float4(vlo[0], vlo[1], vlo[2], vlo[3]);
        *reinterpret_cast<float4*>(dst + m.v_off + half) =
            make_float4(vhi[0], vhi[1], vhi[2], vhi[3]);
      } else {
        dst[0] = klo[0];
        dst[half] = khi[0];
        dst[m.v_off] = vlo[0];
        dst[m.v_off + half] = vhi[0];
      }
    } else if constexpr (VEC == 4) {
      *reinterpret_cast<float4*>(dst) = ld4(K + src);
      *reinterpret_cast<float4*>(dst + m.v_off) = ld4(V + src);
    } else {
      dst[0] = K[src];
      dst[m.v_off] = V[src];
    }
  }
}

// ONE: one new row per sequence, written to the RowDesc's append_block (no
// page-table read), while the first threads apply the pending mirror patches
// and copy the row blob.
template <int VEC, class Map, bool ROPE, bool ONE>
__global__ __launch_bounds__(256) void append_kernel(
    Map m, const RowDesc* __restrict__ rows, const float* __restrict__ K,
    const float* __restrict__ V, int32_t n, int32_t kv_dim, int32_t head_dim,
    int64_t total, const double2* __restrict__ cs, PatchArgs pa) {
  if constexpr (ONE) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < pa.n)
      pa.mirror[pa.patches[3 * i] * pa.stride + pa.patches[3 * i + 1]] = pa.patches[3 * i + 2];
    if (i < pa.n_copy) pa.copy_dst[i] = pa.copy_src[i];
  }
  append_elems<VEC, Map, ROPE, ONE>(m, rows, K, V, n, kv_dim, head_dim, total, cs);
}

// Ints passed by value as kernel arguments (array first: 16-byte aligned, so
// RowDesc records in it load as whole vectors).
struct alignas(16) IntChunk {
  int32_t v[kIntChunk];
  int32_t n;
};

// The one-row append with the step's row blob in the kernel arguments
// (blobs of up to kIntChunk ints): descriptors and patches are read from the
// argument copy -- no read of host memory -- and the first threads store the
// blob to blob_dst for the launches that follow and apply the patches
// (n_patch triples from int patch_off of the blob).
template <int VEC, bool ROPE>
__global__ __launch_bounds__(256) void append_inline_kernel(
    PagedMap m, const float* __restrict__ K, const float* __restrict__ V,
    int32_t kv_dim, int32_t head_dim, int64_t total, const double2* __restrict__ cs,
    int32_t* mirror, int64_t stride, int32_t patch_off, int32_t n_patch,
    int32_t* blob_dst, IntChunk b) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n_patch) {
    const int32_t* pt = b.v + patch_off + 3 * i;
    mirror[pt[0] * stride + pt[1]] = pt[2];
  }
  if (i < b.n) blob_dst[i] = b.v[i];
  append_elems<VEC, PagedMap, ROPE, true>(m, reinterpret_cast<const RowDesc*>(b.v), K, V, 1,
                                          kv_dim, head_dim, total, cs);
}

// ---------------------------------------------------------------------------
// Copy-on-append: copy whole blocks (all layers, K and V) src -> dst.
// ---------------------------------------------------------------------------
template <int VEC>
__global__ __launch_bounds__(256) void cow_kernel(float* base,
                                                  const int32_t* __restrict__ pairs,
                                                  int64_t block_floats) {
  const int64_t src = pairs[2 * blockIdx.y];
  const int64_t dst = pairs[2 * blockIdx.y + 1];
  const float* s = base + src * block_floats;
  float* d = base + dst * block_floats;
  const int64_t n = block_floats / VEC;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    if constexpr (VEC == 4) {
      reinterpret_cast<float4*>(d)[e] = reinterpret_cast<const float4*>(s)[e];
    } else {
      d[e] = s[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Decode, head_dim 128, 16-row pages: one 64-lane wave per
// (work item = row x key split, kv head).
//
// Lane layout: lane = 16 * rr + c.  For each page the wave reads the kv
// head's 16 x 128 K tile and V tile once, four positions per load step:
// position 4*i + rr, dims [4c, 4c+4) and [64+4c, 64+4c+4).  Each K/V byte
// is loaded once and used for all GROUP query heads of the kv head (the GQA
// sharing).  Partial dot products are summed over the 16 lanes of a DPP row
// (row16_sum), so every lane of row rr holds the full scores of positions
// 4*i + rr for all GROUP heads.  Each row keeps its own online-softmax state
// (m, l, o) over the positions it sees; the four row states are merged at
// the end of the split with cross-row shuffles.
// ---------------------------------------------------------------------------
// Split merge for one (row, kv head), run by one 64-lane wave:
// out = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - max_s m_s).
// Lanes own split indices for the statistics and head dims (2 each) for the
// weighted sum, which runs over the splits in ascending order.
// One wave merges one head j of the group.
// Partial results of split s of a row live at slot part_base + s, laid out
// [slot][query][head]; a decode row has one query.
__device__ __forceinline__ void merge_head(const AttnArgs& a, int32_t row,
                                           int32_t qi, int32_t head,
                                           int32_t part_base, int32_t nsp,
                                           int lane) {
  constexpr int D = 128;
  constexpr int U = 8;  // split rows loaded together
  const int64_t H = a.n_heads;
  const int64_t SH = (int64_t)a.n_q * H;  // entries per slot
  const int64_t h0 = (int64_t)part_base * SH + (int64_t)qi * H + head;
  const float* obase = a.part_o + h0 * D + 2 * lane;
  // One round of loads before any arithmetic: this lane's split statistics
  // and the first U partial rows (most rows have at most U splits).
  float m_first = kNegInf, l_first = 0.f;
  if (lane < nsp) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (h0 + lane * SH) * 2);
    m_first = ml.x;
    l_first = ml.y;
  }
  float2 ov0[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    ov0[u] = u < nsp ? *reinterpret_cast<const float2*>(obase + (int64_t)u * SH * D)
                     : make_float2(0.f, 0.f);
  float mx = m_first;
  for (int32_t s = lane + 64; s < nsp; s += 64) mx = fmaxf(mx, a.part_ml[(h0 + s * SH) * 2]);
  mx = wave_max(mx);
  float lw = 0.f, o0 = 0.f, o1 = 0.f;
  for (int32_t s0 = 0; s0 < nsp; s0 += 64) {
    const int32_t s = s0 + lane;
    float w = 0.f;
    if (s < nsp) {
      const float ms = s0 == 0 ? m_first : a.part_ml[(h0 + s * SH) * 2];
      const float ls = s0 == 0 ? l_first : a.part_ml[(h0 + s * SH) * 2 + 1];
      w = fast_exp2(ms - mx);
      lw = fmaf(w, ls, lw);
    }
    const int32_t cnt = min(64, nsp - s0);
    const float* base = obase + (int64_t)s0 * SH * D;
    int32_t t = 0;
    if (s0 == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wt = __shfl(w, u);
        if (u < cnt) {
          o0 = fmaf(wt, ov0[u].x, o0);
          o1 = fmaf(wt, ov0[u].y, o1);
        }
      }
      t = min(U, cnt);
    }
    for (; t + U <= cnt; t += U) {
      float2 ov[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        ov[u] = *reinterpret_cast<const float2*>(base + (int64_t)(t + u) * SH * D);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wt = __shfl(w, t + u);
        o0 = fmaf(wt, ov[u].x, o0);
        o1 = fmaf(wt, ov[u].y, o1);
      }
    }
    for (; t < cnt; ++t) {
      const float wt = __shfl(w, t);
      const float2 ov = *reinterpret_cast<const float2*>(base + (int64_t)t * SH * D);
      o0 = fmaf(wt, ov.x, o0);
      o1 = fmaf(wt, ov.y, o1);
    }
  }
  const float L = wave_sum(lw);
  *reinterpret_cast<float2*>(a.out + (((int64_t)row * a.n_q + qi) * H + head) * D +
                             2 * lane) = make_float2(o0 / L, o1 / L);
}

// One wave's work: work item item_idx (a (row, split) pair), kv head kvh;
// lane = this thread's lane in its wave.  DEEP: two pages in flight ahead of
// the one being used instead of one (more registers: one wave per SIMD for
// group 4 and 8); the arithmetic is the same, page by page, so are the bits.
template <int GROUP, class Map, bool DEEP = false>
__device__ __forceinline__ void decode_wave(const Map& m, const AttnArgs& a,
                                            int32_t item_idx, int32_t kvh,
                                            int lane) {
  constexpr int D = 128;
  constexpr int B = 16;
  constexpr int NI = B / 4;
  const int2 item = a.items[item_idx];
  const int32_t row = item.x, split = item.y;
  const RowDesc rd = a.rows[row];
  const int32_t nsp = rd.n_pre + rd.n_splits;  // partial results of the row
  const int32_t slot = rd.part_base + split;
  const int rr = lane >> 4;
  const int c = lane & 15;

  const int32_t total_k = rd.start + 1;
  const int32_t k_begin = rd.k_off + split * rd.split;
  const int32_t k_end = min(total_k, k_begin + rd.split);
  const int32_t p_begin = k_begin / B;
  const int32_t p_end = (k_end + B - 1) / B;

  float qa[GROUP][4], qb[GROUP][4];
  {
    const float* qrow =
        a.Q + ((int64_t)row * a.n_heads + (int64_t)kvh * GROUP) * D;
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const float4 x = ld4(qrow + j * D + 4 * c);
      const float4 y = ld4(qrow + j * D + 64 + 4 * c);
      qa[j][0] = x.x;
      qa[j][1] = x.y;
      qa[j][2] = x.z;
      qa[j][3] = x.w;
      qb[j][0] = y.x;
      qb[j][1] = y.y;
      qb[j][2] = y.z;
      qb[j][3] = y.w;
    }
    if (a.rope) {
      // the query sits at position total_k - 1; dims 4c+e pair with 64+4c+e
      const double2* cr = a.rope + (int64_t)(total_k - 1) * (D / 2) + 4 * c;
      double2 cse[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) cse[e] = cr[e];
#pragma unroll
      for (int j = 0; j < GROUP; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) rotate_pair(qa[j][e], qb[j][e], cse[e]);
    }
#pragma unroll
    for (int j = 0; j < GROUP; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qa[j][e] *= a.qscale;
        qb[j][e] *= a.qscale;
      }
  }

  float mrun[GROUP], lrun[GROUP];
  float oa[GROUP][4], ob[GROUP][4];
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    mrun[j] = kNegInf;
    lrun[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) oa[j][e] = ob[j][e] = 0.f;
  }

  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 kA[NI], kB[NI], vA[NI], vB[NI];
  auto load_page = [&](int32_t p, float4(&ka)[NI], float4(&kb)[NI],
                       float4(&va)[NI], float4(&vb)[NI]) {
    const float* kp = m.page(rd, p, kvh);
    const float* vp = kp + m.v_off;
    const int32_t n_valid = min(B, k_end - p * B);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = 4 * i + rr;
      const int off = t * D + 4 * c;
      if (t < n_valid) {
        ka[i] = ld4_stream(kp + off);
        kb[i] = ld4_stream(kp + off + 64);
        va[i] = ld4_stream(vp + off);
        vb[i] = ld4_stream(vp + off + 64);
      } else {
        ka[i] = kb[i] = va[i] = vb[i] = zero4;
      }
    }
  };

  // scores, online softmax and weighted sum of one page (in registers)
  auto use_page = [&](int32_t p, const float4(&ka)[NI], const float4(&kb)[NI],
                      const float4(&va)[NI], const float4(&vb)[NI]) {
    const int32_t n_valid = min(B, k_end - p * B);
    float s[NI][GROUP];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < GROUP; ++j)
        s[i][j] = row16_sum(dot8(ka[i], kb[i], qa[j], qb[j]));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (4 * i + rr >= n_valid) {
#pragma unroll
        for (int j = 0; j < GROUP; ++j) s[i][j] = kNegInf;
      }
    }
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      float mx = s[0][j];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[i][j]);
      const float m_new = fmaxf(mrun[j], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(mrun[j] - m_use);
      float pr[NI];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pr[i] = fast_exp2(s[i][j] - m_use);
        psum += pr[i];
      }
      lrun[j] = fmaf(lrun[j], alpha, psum);
      mrun[j] = m_new;
      float xa[4], xb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = oa[j][e] * alpha;
        xb[e] = ob[j][e] * alpha;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        xa[0] = fmaf(pr[i], va[i].x, xa[0]);
        xa[1] = fmaf(pr[i], va[i].y, xa[1]);
        xa[2] = fmaf(pr[i], va[i].z, xa[2]);
        xa[3] = fmaf(pr[i], va[i].w, xa[3]);
        xb[0] = fmaf(pr[i], vb[i].x, xb[0]);
        xb[1] = fmaf(pr[i], vb[i].y, xb[1]);
        xb[2] = fmaf(pr[i], vb[i].z, xb[2]);
        xb[3] = fmaf(pr[i], vb[i].w, xb[3]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oa[j][e] = xa[e];
        ob[j][e] = xb[e];
      }
    }

  };

  load_page(p_begin, kA, kB, vA, vB);
  if constexpr (DEEP) {
    // three register pages used in turn: page p + 2 is requested while page
    // p is used
    float4 k1A[NI], k1B[NI], v1A[NI], v1B[NI];
    float4 k2A[NI], k2B[NI], v2A[NI], v2B[NI];
    if (p_begin + 1 < p_end) load_page(p_begin + 1, k1A, k1B, v1A, v1B);
    for (int32_t p = p_begin; p < p_end; p += 3) {
      if (p + 2 < p_end) load_page(p + 2, k2A, k2B, v2A, v2B);
      use_page(p, kA, kB, vA, vB);
      if (p + 1 >= p_end) break;
      if (p + 3 < p_end) load_page(p + 3, kA, kB, vA, vB);
      use_page(p + 1, k1A, k1B, v1A, v1B);
      if (p + 2 >= p_end) break;
      if (p + 4 < p_end) load_page(p + 4, k1A, k1B, v1A, v1B);
      use_page(p + 2, k2A, k2B, v2A, v2B);
    }
  } else {
    for (int32_t p = p_begin; p < p_end; ++p) {
      float4 nkA[NI], nkB[NI], nvA[NI], nvB[NI];
      if (p + 1 < p_end) load_page(p + 1, nkA, nkB, nvA, nvB);
      use_page(p, kA, kB, vA, vB);
      if (p + 1 < p_end) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          kA[i] = nkA[i];
          kB[i] = nkB[i];
          vA[i] = nvA[i];
          vB[i] = nvB[i];
        }
      }
    }
  }

  // Merge the four row states (lanes 16 and 32 apart hold the other rows).
  float Lf[GROUP];
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    float M = fmaxf(mrun[j], __shfl_xor(mrun[j], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    // every split holds at least one key, so M is finite
    const float w = fast_exp2(mrun[j] - M);
    float L = lrun[j] * w;
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    Lf[j] = L;
    mrun[j] = M;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = oa[j][e] * w;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      oa[j][e] = x;
      float y = ob[j][e] * w;
      y += __shfl_xor(y, 16);
      y += __shfl_xor(y, 32);
      ob[j][e] = y;
    }
  }

  // Row rr writes heads j with j % 4 == rr.
  if (nsp == 1) {
    float* orow = a.out + ((int64_t)row * a.n_heads + (int64_t)kvh * GROUP) * D;
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      if ((j & 3) == rr) {
        float4 x, y;
        x.x = oa[j][0] / Lf[j];
        x.y = oa[j][1] / Lf[j];
        x.z = oa[j][2] / Lf[j];
        x.w = oa[j][3] / Lf[j];
        y.x = ob[j][0] / Lf[j];
        y.y = ob[j][1] / Lf[j];
        y.z = ob[j][2] / Lf[j];
        y.w = ob[j][3] / Lf[j];
        *reinterpret_cast<float4*>(orow + j * D + 4 * c) = x;
        *reinterpret_cast<float4*>(orow + j * D + 64 + 4 * c) = y;
      }
    }
  } else {
    const int64_t hbase = (int64_t)slot * a.n_heads + (int64_t)kvh * GROUP;
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      if ((j & 3) == rr) {
        float* po = a.part_o + (hbase + j) * D;
        st4_stream(po + 4 * c, make_float4(oa[j][0], oa[j][1], oa[j][2], oa[j][3]));
        st4_stream(po + 64 + 4 * c, make_float4(ob[j][0], ob[j][1], ob[j][2], ob[j][3]));
        if (c == 0) {
          __builtin_nontemporal_store(mrun[j], a.part_ml + (hbase + j) * 2 + 0);
          __builtin_nontemporal_store(Lf[j], a.part_ml + (hbase + j) * 2 + 1);
        }
      }
    }
  }
}

template <int GROUP, class Map, bool DEEP>
__global__ __launch_bounds__(64) void decode_fast_kernel(Map m, AttnArgs a) {
  const int32_t item_idx = blockIdx.x / a.n_kv_heads;
  decode_wave<GROUP, Map, DEEP>(m, a, item_idx, blockIdx.x - item_idx * a.n_kv_heads,
                                threadIdx.x);
}

// Split merge kernel: one wave per (row, query, query head) of a row with
// splits, four heads per workgroup.  A separate launch (rather than the last
// split merging in place) keeps the partials coherent across XCDs through
// the kernel boundary; an in-kernel merge needs a device-scope release per
// split, which costs more than this launch.
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int32_t quads = (a.n_heads + 3) / 4;
  const int32_t rq = blockIdx.x / quads;  // row * n_q + query
  const int32_t head = (blockIdx.x - rq * quads) * 4 + (threadIdx.x >> 6);
  const int32_t row = rq / a.n_q;
  const int32_t qi = rq - row * a.n_q;
  const RowDesc rd = a.rows[row];
  const int32_t nsp = rd.n_pre + rd.n_splits;
  if (nsp <= 1 || head >= a.n_heads) return;
  merge_head(a, row, qi, head, rd.part_base - rd.n_pre, nsp, threadIdx.x & 63);
}

// ---------------------------------------------------------------------------
// Multi-row MFMA attention engine (FP32 MFMA 16x16x4, head_dim 128, 16-row
// pages), used by the multi-query decode kernel.  A
// workgroup of NB waves runs 16 NB query rows of one kv head over one key
// range; each wave owns 16 rows (lane l: row l%16).
//
// 16x16x4 operand/result layout: lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; accumulator r of lane l is D[4*(l/16) + r][l%16].
// Scores are computed transposed, S^T[key][row] = K Q^T, and the output as
// O^T[dim][row] = V^T P^T, so both leave each lane with one row's values:
// the softmax statistics and the rescale of O are lane-local, replicated
// over the four lanes l%16 + 16m.
//
// Pages are read in row layout -- lane (m, c) = (l/16, l%16) loads positions
// 4i + m, dims [4c, 4c+4) and [64+4c, 64+4c+4): four 256-byte runs per
// load -- which is directly the A operand of O^T: PV step s contracts over
// key 4s + m, and output block b = 4 half + e gives MFMA row c the dim
// 64 half + 4c + e.  The K operand needs one key per lane, so K goes through
// LDS: lane (c, m) reads key sigma(c) = 4 (c % 4) + c / 4 at dims 16t + 4m
// (score step 4t + e contracts over dim 16t + 4m + e, the order of the Q
// operand qv[t]), which makes score accumulator r of lane group m the score
// of key 4r + m -- the key PV step r needs from that lane.
// One wave keeps V in registers and only K in LDS (no barrier: a wave's LDS
// accesses are in order).  Several waves split each page's loads and share K
// and V through one LDS tile: a barrier after the tile is read, the next page
// stored, a barrier before it is read.
// ---------------------------------------------------------------------------
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f4_at(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

constexpr int kMqKS = 132;  // padded LDS row strides of the K / V tiles
constexpr int kMqVS = 136;

// One K tile (and, for several waves, one V tile) per workgroup: a single
// buffer keeps the two-wave form at 17 KB, so three such workgroups fit a CU
// beside their registers.
template <int NB>
struct MqLds {
  float K[1][16 * kMqKS];
  float V[1][NB == 1 ? 4 : 16 * kMqVS];
};

// Q operand of one row: qp points at the row's head vector; dims
// 16t + 4mq .. +3 land in qv[t], turned at q_pos when a rotary table is set,
// then scaled (base-2 score units).
__device__ __forceinline__ void mq_load_q(const float* qp, bool valid, int mq,
                                          const double2* rope, int32_t q_pos,
                                          float qscale, float4 (&qv)[8]) {
  constexpr int D = 128;
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int t = 0; t < 8; ++t) qv[t] = valid ? ld4(qp + 16 * t + 4 * mq) : zero4;
  if (rope) {
    // dims 16t + 4mq + e (t < 4) pair with the same dims + 64 (t + 4)
    const double2* cr = rope + (int64_t)q_pos * (D / 2) + 4 * mq;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      rotate_pair(qv[t].x, qv[t + 4].x, cr[16 * t + 0]);
      rotate_pair(qv[t].y, qv[t + 4].y, cr[16 * t + 1]);
      rotate_pair(qv[t].z, qv[t + 4].z, cr[16 * t + 2]);
      rotate_pair(qv[t].w, qv[t + 4].w, cr[16 * t + 3]);
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    qv[t].x *= qscale;
    qv[t].y *= qscale;
    qv[t].z *= qscale;
    qv[t].w *= qscale;
  }
}

// Keys [k_begin, k_end) of the pages of rd, kv head kvh; keys above q_pos
// are masked.  Updates this lane's row state (Ot, m_run, l_run).
template <int NB, class Map>
__device__ __forceinline__ void mq_attend(const Map& m, const RowDesc& rd,
                                          int32_t kvh, int32_t k_begin,
                                          int32_t k_end, int32_t q_pos,
                                          const float4 (&qv)[8], floatx4 (&Ot)[8],
                                          float& m_run, float& l_run,
                                          MqLds<NB>& sh) {
  constexpr int D = 128;
  constexpr int B = 16;
  constexpr int KS = kMqKS;
  constexpr int VS = kMqVS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int mq = lane >> 4;
  const int sig = 4 * (c16 & 3) + (c16 >> 2);
  const int32_t p_begin = k_begin / B;
  const int32_t p_end = (k_end + B - 1) / B;
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);

  // positions 4i + mq of page p for i in [i0, i0 + NI), row layout; rows
  // past k_end load zeros (masked scores; zero V keeps 0 * V finite)
  auto load_rows = [&](int32_t p, int i0, auto& ka, auto& kb, auto& va, auto& vb) {
    constexpr int NI = sizeof(ka) / sizeof(float4);
    const float* kp = m.page(rd, p, kvh);
    const float* vp = kp + m.v_off;
    const int32_t n_valid = min(B, k_end - p * B);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int key = 4 * (i0 + j) + mq;
      const int off = key * D + 4 * c16;
      if (key < n_valid) {
        ka[j] = ld4_stream(kp + off);
        kb[j] = ld4_stream(kp + off + 64);
        va[j] = ld4_stream(vp + off);
        vb[j] = ld4_stream(vp + off + 64);
      } else {
        ka[j] = kb[j] = va[j] = vb[j] = zero4;
      }
    }
  };
  auto scores = [&](const float* Kt) {
    floatx4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 kf = *reinterpret_cast<const float4*>(&Kt[sig * KS + 16 * t + 4 * mq]);
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.x, qv[t].x, S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.y, qv[t].y, S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.z, qv[t].z, S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.w, qv[t].w, S, 0, 0, 0);
    }
    return S;
  };
  // mask, online softmax, rescale of O; S becomes P (accumulator r: key
  // p*16 + 4r + mq)
  auto softmax_page = [&](floatx4& S, int32_t p) {
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t key = p * B + 4 * r + mq;
      if (!(key < k_end && key <= q_pos)) S[r] = kNegInf;
      mx = fmaxf(mx, S[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      S[r] = fast_exp2(S[r] - m_use);
      ps += S[r];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = fmaf(l_run, alpha, ps);
    m_run = m_new;
    // alpha is exactly 1 for a row whose maximum did not move: skip the
    // rescale when that holds for every row of the wave
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < 8; ++b) Ot[b] *= alpha;
    }
  };
  // PV step s: key 4s + mq; va / vb: dims 4c + e and 64 + 4c + e
  auto pv_step = [&](const floatx4& P, int s, const float4& va, const float4& vb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Ot[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(va, e), P[s], Ot[e], 0, 0, 0);
      Ot[4 + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(vb, e), P[s], Ot[4 + e], 0, 0, 0);
    }
  };

  if constexpr (NB == 1) {
    float* Ks = sh.K[0];
    float4 kA[4], kB[4], vA[4], vB[4];
    load_rows(p_begin, 0, kA, kB, vA, vB);
    for (int32_t p = p_begin; p < p_end; ++p) {
      float4 nkA[4], nkB[4], nvA[4], nvB[4];
      if (p + 1 < p_end) load_rows(p + 1, 0, nkA, nkB, nvA, nvB);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * i + mq;
        *reinterpret_cast<float4*>(&Ks[key * KS + 4 * c16]) = kA[i];
        *reinterpret_cast<float4*>(&Ks[key * KS + 64 + 4 * c16]) = kB[i];
      }
      floatx4 S = scores(Ks);
      softmax_page(S, p);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) pv_step(S, s2, vA[s2], vB[s2]);
      if (p + 1 < p_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kA[i] = nkA[i];
          kB[i] = nkB[i];
          vA[i] = nvA[i];
          vB[i] = nvB[i];
        }
      }
    }
  } else {
    // wave w loads positions 4i + mq for i in [w NI, (w + 1) NI)
    constexpr int NI = 4 / NB;
    float4 kA[NI], kB[NI], vA[NI], vB[NI];
    auto store_part = [&](int buf) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int key = 4 * (NI * wave + j) + mq;
        *reinterpret_cast<float4*>(&sh.K[buf][key * KS + 4 * c16]) = kA[j];
        *reinterpret_cast<float4*>(&sh.K[buf][key * KS + 64 + 4 * c16]) = kB[j];
        *reinterpret_cast<float4*>(&sh.V[buf][key * VS + 4 * c16]) = vA[j];
        *reinterpret_cast<float4*>(&sh.V[buf][key * VS + 64 + 4 * c16]) = vB[j];
      }
    };
    load_rows(p_begin, NI * wave, kA, kB, vA, vB);
    store_part(0);
    __syncthreads();
    for (int32_t p = p_begin; p < p_end; ++p) {
      if (p + 1 < p_end) load_rows(p + 1, NI * wave, kA, kB, vA, vB);
      floatx4 S = scores(sh.K[0]);
      softmax_page(S, p);
      // take this page's V operands, then let the tile be refilled with the
      // next page while the PV products run
      const float* Vt = sh.V[0];
      float4 vva[4], vvb[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        vva[s2] = *reinterpret_cast<const float4*>(&Vt[(4 * s2 + mq) * VS + 4 * c16]);
        vvb[s2] = *reinterpret_cast<const float4*>(&Vt[(4 * s2 + mq) * VS + 64 + 4 * c16]);
      }
      __syncthreads();
      if (p + 1 < p_end) store_part(0);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) pv_step(S, s2, vva[s2], vvb[s2]);
      __syncthreads();
    }
  }
}

// Row result: accumulator r of block 4 half + e is dim 64 half + 16 mq +
// 4r + e.  dst points at the row's head vector; values are divided by L.
__device__ __forceinline__ void mq_store(float* dst, int mq,
                                         const floatx4 (&Ot)[8], float L) {
  dst += 16 * mq;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    *reinterpret_cast<float4*>(dst + 4 * r) =
        make_float4(Ot[0][r] / L, Ot[1][r] / L, Ot[2][r] / L, Ot[3][r] / L);
    *reinterpret_cast<float4*>(dst + 64 + 4 * r) =
        make_float4(Ot[4][r] / L, Ot[5][r] / L, Ot[6][r] / L, Ot[7][r] / L);
  }
}
__device__ __forceinline__ void mq_store_partial(float* dst, int mq,
                                                 const floatx4 (&Ot)[8]) {
  dst += 16 * mq;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    *reinterpret_cast<float4*>(dst + 4 * r) =
        make_float4(Ot[0][r], Ot[1][r], Ot[2][r], Ot[3][r]);
    *reinterpret_cast<float4*>(dst + 64 + 4 * r) =
        make_float4(Ot[4][r], Ot[5][r], Ot[6][r], Ot[7][r]);
  }
}

// ---------------------------------------------------------------------------
// Multi-query decode (a few new rows per sequence, e.g. verifying drafted
// tokens; offset-causal): one workgroup per (work item = row x key split,
// kv head) runs all n_q x group query rows of its kv head (row rho =
// query * group + head in group), NB = 1 or 2 waves of 16 rows.
// ---------------------------------------------------------------------------
template <int NB, class Map>
__global__ __launch_bounds__(64 * NB)
__attribute__((amdgpu_waves_per_eu(NB == 1 ? 2 : 3, NB == 1 ? 2 : 3)))
void verify_mfma_kernel(Map m, AttnArgs a, int32_t group) {
  constexpr int D = 128;
  __shared__ MqLds<NB> sh;
  const int32_t G = a.n_kv_heads;
  const int32_t item_idx = blockIdx.x / G;
  const int32_t kvh = blockIdx.x - item_idx * G;
  const int2 item = a.items[item_idx];
  const int32_t row = item.x, split = item.y;
  const RowDesc rd = a.rows[row];
  const int32_t nsp = rd.n_pre + rd.n_splits;
  const int32_t slot = rd.part_base + split;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int mq = lane >> 4;
  const int32_t n_q = a.n_q;
  const int32_t total_k = rd.start + n_q;
  const int32_t k_begin = rd.k_off + split * rd.split;
  const int32_t k_end = min(total_k, k_begin + rd.split);

  // This lane's query row; rows past n_q * group hold zeros, see every key
  // of the split and are not written.
  const int32_t rho = 16 * wave + (lane & 15);
  const bool valid = rho < n_q * group;
  const int32_t qi = valid ? rho / group : n_q - 1;
  const int32_t hj = valid ? rho - qi * group : 0;
  const int32_t q_pos = rd.start + qi;  // total_k - n_q + qi
  const int64_t qrow = ((int64_t)row * n_q + qi) * a.n_heads + (int64_t)kvh * group + hj;
  float4 qv[8];
  mq_load_q(a.Q + qrow * D, valid, mq, a.rope, q_pos, a.qscale, qv);

  floatx4 Ot[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) Ot[b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  mq_attend<NB>(m, rd, kvh, k_begin, k_end, a.causal ? q_pos : INT32_MAX, qv, Ot,
                m_run, l_run, sh);

  if (!valid) return;
  if (nsp == 1) {
    mq_store(a.out + qrow * D, mq, Ot, l_run);
  } else {
    const int64_t e = ((int64_t)slot * n_q + qi) * a.n_heads + kvh * group + hj;
    mq_store_partial(a.part_o + e * D, mq, Ot);
    if (mq == 0) {
      a.part_ml[e * 2 + 0] = m_run;
      a.part_ml[e * 2 + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic attention (any head_dim, group, page size; decode or prefill): one
// wave per (query row, kv head) over all its visible keys.  Lanes take 64
// keys at a time for the scores; for the weighted sum they take dims.
// ---------------------------------------------------------------------------
constexpr int kGenericMaxGroup = 16;

template <class Map>
__global__ __launch_bounds__(64) void generic_kernel(Map m, AttnArgs a,
                                                     int32_t group) {
  extern __shared__ float sh[];
  const int32_t D = a.head_dim;
  const int32_t G = a.n_kv_heads;
  const int32_t item_idx = blockIdx.x / G;  // = row * n_q + query
  const int32_t kvh = blockIdx.x - item_idx * G;
  const int32_t row = item_idx / a.n_q;
  const int32_t qi = item_idx - row * a.n_q;
  const RowDesc rd = a.rows[row];
  const int lane = threadIdx.x;
  float* q_sh = sh;                // [group][D]
  float* o_sh = q_sh + group * D;  // [group][D]
  float* p_sh = o_sh + group * D;  // [group][64]

  const int32_t total_k = rd.start + a.n_q;
  const int32_t q_pos = total_k - a.n_q + qi;
  const int32_t vis = a.causal ? q_pos + 1 : total_k;
  const int32_t k_begin = 0;
  const int32_t k_end = vis;
  const int64_t out_row = item_idx;

  const float* qrow = a.Q + (out_row * a.n_heads + (int64_t)kvh * group) * D;
  const int32_t half = D / 2;
  for (int32_t e = lane; e < group * D; e += 64) {
    float x = qrow[e];
    if (a.rope) {
      // rotate the pair (i, i + half) this element belongs to at q_pos
      const int32_t d = e % D;
      const int32_t i = d < half ? d : d - half;
      float lo = qrow[e - d + i], hi = qrow[e - d + i + half];
      rotate_pair(lo, hi, a.rope[(int64_t)q_pos * half + i]);
      x = d < half ? lo : hi;
    }
    q_sh[e] = x * a.qscale;
    o_sh[e] = 0.f;
  }
  __syncthreads();

  float mrun[kGenericMaxGroup], lrun[kGenericMaxGroup], alpha[kGenericMaxGroup];
#pragma unroll
  for (int j = 0; j < kGenericMaxGroup; ++j) {
    mrun[j] = kNegInf;
    lrun[j] = 0.f;
    alpha[j] = 1.f;
  }

  const int32_t B = m.block_size;
  for (int32_t c0 = k_begin; c0 < k_end; c0 += 64) {
    const int32_t key = c0 + lane;
    const bool valid = key < k_end;
    const float* kr = valid ? m.page(rd, key / B, kvh) + (int64_t)(key % B) * D
                            : nullptr;
#pragma unroll
    for (int j = 0; j < kGenericMaxGroup; ++j) {
      if (j < group) {
        float s = kNegInf;
        if (valid) {
          float acc = 0.f;
          for (int32_t d = 0; d < D; ++d) acc = fmaf(q_sh[j * D + d], kr[d], acc);
          s = acc;
        }
        const float m_new = fmaxf(mrun[j], wave_max(s));
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float p = valid ? fast_exp2(s - m_use) : 0.f;
        alpha[j] = fast_exp2(mrun[j] - m_use);
        lrun[j] = fmaf(lrun[j], alpha[j], wave_sum(p));
        mrun[j] = m_new;
        p_sh[j * 64 + lane] = p;
      }
    }
    __syncthreads();
    const int32_t n_here = min(64, k_end - c0);
    for (int32_t d = lane; d < D; d += 64) {
#pragma unroll
      for (int j = 0; j < kGenericMaxGroup; ++j) {
        if (j < group) {
          float acc = o_sh[j * D + d] * alpha[j];
          for (int32_t k = 0; k < n_here; ++k) {
            const int32_t kk = c0 + k;
            const float* vr = m.page(rd, kk / B, kvh) + m.v_off +
                              (int64_t)(kk % B) * D;
            acc = fmaf(p_sh[j * 64 + k], vr[d], acc);
          }
          o_sh[j * D + d] = acc;
        }
      }
    }
    __syncthreads();
  }

  float* orow = a.out + (out_row * a.n_heads + (int64_t)kvh * group) * D;
  for (int32_t d = lane; d < D; d += 64) {
#pragma unroll
    for (int j = 0; j < kGenericMaxGroup; ++j)
      if (j < group) orow[j * D + d] = o_sh[j * D + d] / lrun[j];
  }
}

// ---------------------------------------------------------------------------
// Page-table mirror patches: mirror[seq * stride + page] = block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void patch_kernel(int32_t* mirror,
                                                    const int32_t* __restrict__ p,
                                                    int32_t n, int64_t stride) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) mirror[p[3 * i] * stride + p[3 * i + 1]] = p[3 * i + 2];
}

// ---------------------------------------------------------------------------
// Chunked prefill on FP32 MFMA (v_mfma_f32_32x32x2_f32), head_dim 128, GQA
// group GROUP in {1, 2, 4, 8}, 16-row pages.
//
// Workgroup = 4 waves of one (row, kv head).  Each wave owns 32 MFMA rows =
// 32 / GROUP queries x the GROUP heads of the group (row = GROUP*query +
// head), so one K/V tile feeds every head of the group; a workgroup covers
// prefill_q_tile(GROUP) = 128 / GROUP queries.  Keys are processed in tiles
// of 32 (two pages) staged in LDS by the whole workgroup.
//
//   S^T[key][row] = sum_d K[key][d] Q[row][d]     (64 MFMAs, K=2 each)
//   mask (offset-causal), online softmax per row
//   O^T[d][row]  += sum_key V[key][d] P[row][key]  (4 x 16 MFMAs)
//
// 32x32 MFMA operand/result layout: lane l supplies A[l%32][l/32] and
// B[l/32][l%32]; accumulator r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
// Computing S and O transposed leaves each lane with one row's scores and
// output, so the softmax statistics, the rescale of O and the final divide
// are lane-local; the contraction index of the PV product is permuted to
// match the score accumulators (key 8*(s/4) + 4*h + s%4 at step s).
// ---------------------------------------------------------------------------
typedef float floatx16 __attribute__((ext_vector_type(16)));

// PREFIX = true is the shared-prefix form of the same kernel (shared-prefix
// decode): one workgroup per (prefix item = group x kPrefixSplit prefix keys
// x block of 128 query rows, kv head); its MFMA rows are (member, head)
// pairs of the group's members -- the batch rows that share the prefix, one
// new query each -- over the prefix keys of the split, read through the
// first member's page table; nothing is masked (every prefix key precedes
// each member's new row) and each row's unnormalised state goes to its
// prefix partial slot for merge_kernel.
constexpr int kPfKT = 32;     // keys per tile
constexpr float kLazyMax = 8.f;  // lazy-rescale threshold (base-2 score units)
constexpr int kPfKSTR = 132;  // padded LDS row strides (bank spread)
constexpr int kPfVSTR = 136;
// two K/V tile buffers: tile t+1 is stored while tile t is read
struct PrefillLds {
  float Ks2[2][kPfKT * kPfKSTR];
  float Vs2[2][kPfKT * kPfVSTR];
};

// One workgroup's work (all 256 threads), workgroup number bid.
template <int GROUP, bool PREFIX, class Map>
__device__ __forceinline__ void prefill_block(const Map& m, const AttnArgs& a,
                                              int32_t n_qt, int32_t n_wg,
                                              int32_t bid, PrefillLds& sh) {
  constexpr int D = 128;
  constexpr int QPW = 32 / GROUP;  // queries per wave
  constexpr int KT = kPfKT;
  constexpr int KSTR = kPfKSTR;
  constexpr int VSTR = kPfVSTR;
  auto& Ks2 = sh.Ks2;
  auto& Vs2 = sh.Vs2;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int32_t G = a.n_kv_heads;
  const int32_t jh = lr % GROUP;  // head of the group of this lane's MFMA row

  // What this workgroup runs: the pages of rd for kv head kvh, keys
  // [k_first, k_lim); this lane's query row (q_row indexes Q and out rows,
  // q_pos is its position, keys above mask_pos are masked); the keys wave w
  // needs at all (w_lim).
  RowDesc rd;
  int32_t kvh, k_first, k_lim, q_row, q_pos, mask_pos, w_lim;
  int32_t w_mask_min;  // smallest mask position of the wave's rows
  bool row_valid;
  int64_t slot = 0;  // PREFIX: the row's partial slot
  if constexpr (!PREFIX) {
    // Keep all query tiles of one (row, kv head) on one XCD (they share K/V).
    const int32_t b = bid;
    const int32_t Lw = (n_wg % 8 == 0) ? (b % 8) * (n_wg / 8) + b / 8 : b;
    const int32_t row = Lw / (G * n_qt);
    const int32_t rem = Lw - row * G * n_qt;
    kvh = rem / n_qt;
    // longest query tiles (most visible keys) first: the short ones fill the
    // slots that free up last
    const int32_t qt = n_qt - 1 - (rem - kvh * n_qt);
    rd = a.rows[row];
    const int32_t n_q = a.n_q;
    const int32_t total_k = rd.start + n_q;
    const int32_t q0 = qt * (4 * QPW);
    const int32_t qi = q0 + QPW * w + lr / GROUP;
    row_valid = qi < n_q;
    q_pos = row_valid ? total_k - n_q + qi : total_k - 1;
    q_row = row * n_q + (row_valid ? qi : 0);
    mask_pos = a.causal ? q_pos : INT32_MAX;
    k_first = 0;
    const int32_t q_last = min(q0 + 4 * QPW, n_q) - 1;
    k_lim = a.causal ? total_k - n_q + q_last + 1 : total_k;
    const int32_t wq_first = q0 + QPW * w;
    const int32_t wq_last = min(q0 + QPW * w + QPW - 1, n_q - 1);
    w_lim = (wq_first > wq_last) ? 0 : (a.causal ? total_k - n_q + wq_last + 1 : total_k);
    w_mask_min = a.causal ? total_k - n_q + wq_first : INT32_MAX;
  } else {
    const int32_t item = bid / G;
    kvh = bid - item * G;
    const int4 it = reinterpret_cast<const int4*>(a.pre_items)[item];
    const int4 gd = reinterpret_cast<const int4*>(a.groups)[it.x];
    k_first = it.y * kPrefixSplit;
    k_lim = min(gd.w, k_first + kPrefixSplit);
    const int32_t m0 = it.z * (4 * QPW);
    const int32_t mi = m0 + QPW * w + lr / GROUP;
    row_valid = mi < gd.z;
    const int32_t mrow = a.members[gd.y + (row_valid ? mi : 0)];
    const RowDesc md = a.rows[mrow];
    rd = a.rows[gd.x];
    q_row = mrow;
    q_pos = md.start;
    mask_pos = INT32_MAX;
    w_mask_min = INT32_MAX;
    w_lim = (m0 + QPW * w < gd.z) ? k_lim : 0;
    slot = md.part_base - md.n_pre + it.y;
  }

  float4 qreg[16];
  {
    const float* qp =
        a.Q + ((int64_t)q_row * a.n_heads + kvh * GROUP + jh) * D + 4 * h;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      qreg[t] = row_valid ? ld4(qp + 8 * t) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.rope) {
      // qreg[t] holds dims 8t+4h .. 8t+4h+3; for t < 8 they pair with
      // qreg[t + 8] (dims + 64).  Invalid rows hold zeros and stay zero.
      const double2* cr = a.rope + (int64_t)q_pos * (D / 2) + 4 * h;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        rotate_pair(qreg[t].x, qreg[t + 8].x, cr[8 * t + 0]);
        rotate_pair(qreg[t].y, qreg[t + 8].y, cr[8 * t + 1]);
        rotate_pair(qreg[t].z, qreg[t + 8].z, cr[8 * t + 2]);
        rotate_pair(qreg[t].w, qreg[t + 8].w, cr[8 * t + 3]);
      }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      qreg[t].x *= a.qscale;
      qreg[t].y *= a.qscale;
      qreg[t].z *= a.qscale;
      qreg[t].w *= a.qscale;
    }
  }

  const int32_t t_first = k_first / KT;
  const int32_t n_tiles = (k_lim + KT - 1) / KT;

  floatx16 O0 = {}, O1 = {}, O2 = {}, O3 = {};
  float m_run = kNegInf;
  float l_run = 0.f;

  // tile loader: float4 index tid + 256*u, u < 4: key tid/32 + 8u, dims 4*(tid%32)
  const int ld_key = tid >> 5;
  const int ld_c = (tid & 31) * 4;
  float4 kr[4], vr[4];
  auto load_tile = [&](int32_t t) {
    const int32_t k0 = t * KT;
    const int32_t pg = k0 / 16;
    const float* p0 = m.page(rd, pg, kvh);
    const float* p1 = (k0 + 16 < k_lim) ? m.page(rd, pg + 1, kvh) : p0;
    if (k0 + KT <= k_lim) {
      // whole tile present: plain loads
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = ld_key + 8 * u;
        const float* base = (u < 2) ? p0 : p1;
        const int off = (key & 15) * D + ld_c;
        kr[u] = ld4(base + off);
        vr[u] = ld4(base + m.v_off + off);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = ld_key + 8 * u;
      const float* base = (u < 2) ? p0 : p1;
      const int off = (key & 15) * D + ld_c;
      if (k0 + key < k_lim) {
        kr[u] = ld4(base + off);
        vr[u] = ld4(base + m.v_off + off);
      } else {
        kr[u] = vr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = ld_key + 8 * u;
      *reinterpret_cast<float4*>(&Ks2[buf][key * KSTR + ld_c]) = kr[u];
      *reinterpret_cast<float4*>(&Vs2[buf][key * VSTR + ld_c]) = vr[u];
    }
  };

  load_tile(t_first);
  store_tile(0);
  __syncthreads();
  for (int32_t t = t_first; t < n_tiles; ++t) {
    const int buf = (t - t_first) & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const float* Ks = Ks2[buf];
    const float* Vs = Vs2[buf];
    const int32_t k0 = t * KT;
    if (k0 < w_lim) {
      floatx16 S = {};
      if constexpr (PREFIX) {
        // one workgroup per CU here (one wave per SIMD): two independent
        // accumulation chains (even / odd dims of each group of four),
        // summed at the end, so the matrix pipe never waits on the
        // previous MFMA's result
        floatx16 S2 = {};
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float4 kf = *reinterpret_cast<const float4*>(&Ks[lr * KSTR + 8 * u + 4 * h]);
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qreg[u].x, S, 0, 0, 0);
          S2 = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qreg[u].y, S2, 0, 0, 0);
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qreg[u].z, S, 0, 0, 0);
          S2 = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qreg[u].w, S2, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] += S2[r];
      } else {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float4 kf = *reinterpret_cast<const float4*>(&Ks[lr * KSTR + 8 * u + 4 * h]);
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qreg[u].x, S, 0, 0, 0);
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qreg[u].y, S, 0, 0, 0);
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qreg[u].z, S, 0, 0, 0);
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qreg[u].w, S, 0, 0, 0);
        }
      }
      // mask and row max: this lane holds row lr, keys k0 + 8*(r/4) + 4*h + r%4
      float mx = kNegInf;
      if (k0 + KT <= k_lim && k0 + KT - 1 <= w_mask_min) {
        // every key of the tile is visible to every row of the wave
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (!(key < k_lim && key <= mask_pos)) S[r] = kNegInf;
          mx = fmaxf(mx, S[r]);
        }
      }
      // Lazy rescale: the reference maximum m_run of a row moves only when
      // a score exceeds it by more than kLazyMax (base-2 units); below that
      // the tile's weights are taken against the old reference (each at
      // most 2^kLazyMax).  O and l share the reference, so O / l is the
      // softmax-weighted sum either way.  The test is wave-uniform; in it
      // the two lanes of a row (h = 0, 1) agree on the row maximum.  The
      // first tile always moves it (m_run starts at -inf and every row
      // sees a key of its first tile: causal rows see key 0 onwards).
      if (__ballot(mx > m_run + kLazyMax)) {
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
        // every O^T block keeps row lr in this lane: the rescale is
        // lane-local
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          O0[r] *= alpha;
          O1[r] *= alpha;
          O2[r] *= alpha;
          O3[r] *= alpha;
        }
      }
      // this lane's keys only: the two halves of a row's sum are added once,
      // after the last tile
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S[r] = fast_exp2(S[r] - m_run);
        ps += S[r];
      }
      l_run += ps;
      // O^T = V^T P^T: A = V^T (lane: dim 32b + lr, key of step s), B = P^T
      // (lane: row lr, the same key -- score accumulator s)
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int key = 8 * (s >> 2) + 4 * h + (s & 3);
        const float* vrow = &Vs[key * VSTR + lr];
        O0 = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[0], S[s], O0, 0, 0, 0);
        O1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32], S[s], O1, 0, 0, 0);
        O2 = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[64], S[s], O2, 0, 0, 0);
        O3 = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[96], S[s], O3, 0, 0, 0);
      }
    }
    // The other buffer was last read in iteration t-1, which ended with a
    // barrier, so it can be refilled now; one barrier per tile.
    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Store: this lane holds row lr (query or member, head jh); accumulator r
  // of block b is dim 32b + 8(r/4) + 4h + r%4.  Prefill divides by the row
  // sum; the prefix form writes the unnormalised state of its key range.
  l_run += __shfl_xor(l_run, 32);
  if (!row_valid) return;
  const int64_t e = PREFIX ? slot * a.n_heads + kvh * GROUP + jh
                           : (int64_t)q_row * a.n_heads + kvh * GROUP + jh;
  float* op = (PREFIX ? a.part_o : a.out) + e * D + 4 * h;
  const float L = PREFIX ? 1.f : l_run;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    *reinterpret_cast<float4*>(op + 8 * g) =
        make_float4(O0[4 * g] / L, O0[4 * g + 1] / L, O0[4 * g + 2] / L, O0[4 * g + 3] / L);
    *reinterpret_cast<float4*>(op + 32 + 8 * g) =
        make_float4(O1[4 * g] / L, O1[4 * g + 1] / L, O1[4 * g + 2] / L, O1[4 * g + 3] / L);
    *reinterpret_cast<float4*>(op + 64 + 8 * g) =
        make_float4(O2[4 * g] / L, O2[4 * g + 1] / L, O2[4 * g + 2] / L, O2[4 * g + 3] / L);
    *reinterpret_cast<float4*>(op + 96 + 8 * g) =
        make_float4(O3[4 * g] / L, O3[4 * g + 1] / L, O3[4 * g + 2] / L, O3[4 * g + 3] / L);
  }
  if (PREFIX && h == 0) {
    a.part_ml[e * 2 + 0] = m_run;
    a.part_ml[e * 2 + 1] = l_run;
  }
}

// Two waves per SIMD (two workgroups per CU): the register budget is capped at
// 256 so one workgroup's MFMAs overlap the other's softmax, LDS and barriers.
template <int GROUP, class Map>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(Map m, AttnArgs a, int32_t n_qt, int32_t n_wg) {
  __shared__ PrefillLds sh;
  prefill_block<GROUP, false>(m, a, n_qt, n_wg, blockIdx.x, sh);
}

// Shared-prefix decode in one launch: the first workgroups run four decode
// work items each, one per wave, over the rows' own keys; the last
// n_pre_items * kv heads run the prefix items (prefix mode of the prefill
// work).  The two kinds write disjoint partial slots.  The decode waves use
// no LDS and no barrier; dispatched first, they take one workgroup slot of a
// CU each, which leaves the prefix workgroups spread one per CU (measured
// ~8% faster on the forked batch than prefix workgroups first).
template <int GROUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void shared_decode_kernel(PagedMap m, AttnArgs a) {
  __shared__ PrefillLds sh;
  const int32_t n_pre_wg = a.n_pre_items * a.n_kv_heads;
  const int32_t n_dec_wg = gridDim.x - n_pre_wg;
  if (static_cast<int32_t>(blockIdx.x) >= n_dec_wg) {
    prefill_block<GROUP, true>(m, a, 0, 0, blockIdx.x - n_dec_wg, sh);
    return;
  }
  const int32_t wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= a.n_items * a.n_kv_heads) return;
  const int32_t item_idx = wv / a.n_kv_heads;
  decode_wave<GROUP>(m, a, item_idx, wv - item_idx * a.n_kv_heads, threadIdx.x & 63);
}

template <class Map, bool ONE>
hipError_t append_impl(const Map& m, const RowDesc* rows, const float* K,
                       const float* V, int32_t M, int32_t n, int32_t kv_dim,
                       int32_t head_dim, const double2* cs, const PatchArgs& pa,
                       hipStream_t st) {
  const bool rope = cs != nullptr;
  if (rope && head_dim % 2 != 0) return hipErrorInvalidValue;
  const int32_t span = rope ? head_dim / 2 : head_dim;
  const bool vec = (span % 4 == 0);
  const int64_t total = (int64_t)M * n * (rope ? kv_dim / 2 : kv_dim) / (vec ? 4 : 1);
  const int64_t want = (std::max<int64_t>({total, pa.n, pa.n_copy}) + 255) / 256;
  const int grid = static_cast<int>(want < 65536 ? (want > 0 ? want : 1) : 65536);
  if (ONE && ((int64_t)grid * 256 < pa.n || (int64_t)grid * 256 < pa.n_copy))
    return hipErrorInvalidValue;
  if (rope && vec)
    append_kernel<4, Map, true, ONE><<<grid, 256, 0, st>>>(m, rows, K, V, n, kv_dim,
                                                           head_dim, total, cs, pa);
  else if (rope)
    append_kernel<1, Map, true, ONE><<<grid, 256, 0, st>>>(m, rows, K, V, n, kv_dim,
                                                           head_dim, total, cs, pa);
  else if (vec)
    append_kernel<4, Map, false, ONE><<<grid, 256, 0, st>>>(m, rows, K, V, n, kv_dim,
                                                            head_dim, total, cs, pa);
  else
    append_kernel<1, Map, false, ONE><<<grid, 256, 0, st>>>(m, rows, K, V, n, kv_dim,
                                                            head_dim, total, cs, pa);
  return hipGetLastError();
}

template <int GROUP, class Map>
void decode_fast_launch(const Map& m, const AttnArgs& a, bool deep, hipStream_t st) {
  const dim3 grid(a.n_items * a.n_kv_heads);
  if (deep)
    decode_fast_kernel<GROUP, Map, true><<<grid, 64, 0, st>>>(m, a);
  else
    decode_fast_kernel<GROUP, Map, false><<<grid, 64, 0, st>>>(m, a);
}

template <class Map>
hipError_t decode_fast_impl(const Map& m, const AttnArgs& a, int32_t group, bool deep,
                            hipStream_t st) {
  switch (group) {
    case 1: decode_fast_launch<1>(m, a, deep, st); break;
    case 2: decode_fast_launch<2>(m, a, deep, st); break;
    case 4: decode_fast_launch<4>(m, a, deep, st); break;
    case 8: decode_fast_launch<8>(m, a, deep, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class Map>
hipError_t verify_impl(const Map& m, const AttnArgs& a, int32_t group,
                       hipStream_t st) {
  const dim3 grid(a.n_items * a.n_kv_heads);
  const int32_t rows = a.n_q * group;
  if (rows <= 16)
    verify_mfma_kernel<1, Map><<<grid, 64, 0, st>>>(m, a, group);
  else if (rows <= 32)
    verify_mfma_kernel<2, Map><<<grid, 128, 0, st>>>(m, a, group);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t shared_decode_impl(const PagedMap& m, const AttnArgs& a, int32_t group,
                              hipStream_t st) {
  const int64_t waves = (int64_t)a.n_items * a.n_kv_heads;
  const dim3 grid(a.n_pre_items * a.n_kv_heads + (waves + 3) / 4);
  switch (group) {
    case 1: shared_decode_kernel<1><<<grid, 256, 0, st>>>(m, a); break;
    case 2: shared_decode_kernel<2><<<grid, 256, 0, st>>>(m, a); break;
    case 4: shared_decode_kernel<4><<<grid, 256, 0, st>>>(m, a); break;
    case 8: shared_decode_kernel<8><<<grid, 256, 0, st>>>(m, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t merge_impl(const AttnArgs& a, hipStream_t st) {
  merge_kernel<<<a.n_rows * a.n_q * ((a.n_heads + 3) / 4), 256, 0, st>>>(a);
  return hipGetLastError();
}

template <class Map>
hipError_t generic_impl(const Map& m, const AttnArgs& a, int32_t group,
                        hipStream_t st) {
  if (group > kGenericMaxGroup) return hipErrorInvalidValue;
  const size_t lds = sizeof(float) * (2 * (size_t)group * a.head_dim + (size_t)group * 64);
  const dim3 grid(a.n_rows * a.n_q * a.n_kv_heads);
  generic_kernel<Map><<<grid, 64, lds, st>>>(m, a, group);
  return hipGetLastError();
}

template <int GROUP, class Map>
hipError_t prefill_group(const Map& m, const AttnArgs& a, hipStream_t st) {
  constexpr int32_t qt = prefill_q_tile(GROUP);
  const int32_t n_qt = (a.n_q + qt - 1) / qt;
  const int32_t n_wg = a.n_rows * a.n_kv_heads * n_qt;
  prefill_mfma_kernel<GROUP, Map><<<n_wg, 256, 0, st>>>(m, a, n_qt, n_wg);
  return hipGetLastError();
}

template <class Map>
hipError_t prefill_impl(const Map& m, const AttnArgs& a, int32_t group,
                        hipStream_t st) {
  switch (group) {
    case 1: return prefill_group<1>(m, a, st);
    case 2: return prefill_group<2>(m, a, st);
    case 4: return prefill_group<4>(m, a, st);
    case 8: return prefill_group<8>(m, a, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Zero-allocation decode support.  The scratch array is device memory the
// library never allocates at run time: the code object carries it, and each
// GPU gets its own copy when the library's kernels are loaded there.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void write_ints_kernel(int32_t* dst, IntChunk c) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < c.n) dst[i] = c.v[i];
}

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocBlobBytes + kNoAllocPartBytes];

hipError_t noalloc_scratch(void** base) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    addr[dev] = p;
  }
  *base = addr[dev];
  return hipSuccess;
}

hipError_t launch_write_ints(int32_t* dst, const int32_t* src, size_t n, hipStream_t st) {
  IntChunk c;
  for (size_t off = 0; off < n; off += kIntChunk) {
    c.n = static_cast<int32_t>(std::min<size_t>(kIntChunk, n - off));
    std::copy(src + off, src + off + c.n, c.v);
    write_ints_kernel<<<(c.n + 255) / 256, 256, 0, st>>>(dst + off, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_patch(int32_t* mirror, const int32_t* patches, int32_t n,
                        int64_t stride, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  patch_kernel<<<(n + 255) / 256, 256, 0, st>>>(mirror, patches, n, stride);
  return hipGetLastError();
}


hipError_t launch_append(const PagedMap& m, const RowDesc* rows, const float* K,
                         const float* V, int32_t M, int32_t n, int32_t kv_dim,
                         int32_t head_dim, const double2* rope, hipStream_t st) {
  return append_impl<PagedMap, false>(m, rows, K, V, M, n, kv_dim, head_dim, rope,
                                      PatchArgs{}, st);
}
hipError_t launch_append(const ContigMap& m, const RowDesc* rows,
                         const float* K, const float* V, int32_t M, int32_t n,
                         int32_t kv_dim, int32_t head_dim, const double2* rope,
                         hipStream_t st) {
  return append_impl<ContigMap, false>(m, rows, K, V, M, n, kv_dim, head_dim, rope,
                                       PatchArgs{}, st);
}
hipError_t launch_append_one(const PagedMap& m, const RowDesc* rows,
                             const float* K, const float* V, int32_t M,
                             int32_t kv_dim, int32_t head_dim,
                             const double2* rope, const PatchArgs& pa,
                             hipStream_t st) {
  return append_impl<PagedMap, true>(m, rows, K, V, M, 1, kv_dim, head_dim, rope, pa,
                                     st);
}

hipError_t launch_append_inline(const PagedMap& m, const float* K, const float* V,
                                int32_t M, int32_t kv_dim, int32_t head_dim,
                                const double2* rope, int32_t* mirror, int64_t stride,
                                int32_t* blob_dst, const int32_t* blob, int32_t n_blob,
                                int32_t patch_off, int32_t n_patch, hipStream_t st) {
  if (n_blob < 0 || n_blob > kIntChunk || patch_off < 0 ||
      (int64_t)patch_off + 3 * (int64_t)n_patch > n_blob)
    return hipErrorInvalidValue;
  const bool rope_on = rope != nullptr;
  if (rope_on && head_dim % 2 != 0) return hipErrorInvalidValue;
  const int32_t span = rope_on ? head_dim / 2 : head_dim;
  const bool vec = (span % 4 == 0);
  const int64_t total = (int64_t)M * (rope_on ? kv_dim / 2 : kv_dim) / (vec ? 4 : 1);
  const int64_t want = (std::max<int64_t>({total, n_patch, n_blob}) + 255) / 256;
  const int grid = static_cast<int>(want < 65536 ? (want > 0 ? want : 1) : 65536);
  if ((int64_t)grid * 256 < n_blob) return hipErrorInvalidValue;
  IntChunk c;
  c.n = n_blob;
  std::copy(blob, blob + n_blob, c.v);
  if (rope_on && vec)
    append_inline_kernel<4, true><<<grid, 256, 0, st>>>(m, K, V, kv_dim, head_dim, total, rope,
                                                         mirror, stride, patch_off, n_patch,
                                                         blob_dst, c);
  else if (rope_on)
    append_inline_kernel<1, true><<<grid, 256, 0, st>>>(m, K, V, kv_dim, head_dim, total, rope,
                                                         mirror, stride, patch_off, n_patch,
                                                         blob_dst, c);
  else if (vec)
    append_inline_kernel<4, false><<<grid, 256, 0, st>>>(m, K, V, kv_dim, head_dim, total,
                                                          rope, mirror, stride, patch_off,
                                                          n_patch, blob_dst, c);
  else
    append_inline_kernel<1, false><<<grid, 256, 0, st>>>(m, K, V, kv_dim, head_dim, total,
                                                          rope, mirror, stride, patch_off,
                                                          n_patch, blob_dst, c);
  return hipGetLastError();
}

hipError_t launch_cow(float* base, const int32_t* pairs, int32_t n_pairs,
                      int64_t block_floats, hipStream_t st) {
  const bool vec = (block_floats % 4 == 0);
  const int64_t n = block_floats / (vec ? 4 : 1);
  const int64_t want = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(want < 1024 ? want : 1024), n_pairs);
  if (vec)
    cow_kernel<4><<<grid, 256, 0, st>>>(base, pairs, block_floats);
  else
    cow_kernel<1><<<grid, 256, 0, st>>>(base, pairs, block_floats);
  return hipGetLastError();
}

hipError_t launch_decode_fast(const PagedMap& m, const AttnArgs& a,
                              int32_t group, bool deep, hipStream_t st) {
  return decode_fast_impl(m, a, group, deep, st);
}
hipError_t launch_decode_fast(const ContigMap& m, const AttnArgs& a,
                              int32_t group, bool deep, hipStream_t st) {
  return decode_fast_impl(m, a, group, deep, st);
}
hipError_t launch_verify_mfma(const PagedMap& m, const AttnArgs& a,
                              int32_t group, hipStream_t st) {
  return verify_impl(m, a, group, st);
}
hipError_t launch_verify_mfma(const ContigMap& m, const AttnArgs& a,
                              int32_t group, hipStream_t st) {
  return verify_impl(m, a, group, st);
}
hipError_t launch_shared_decode(const PagedMap& m, const AttnArgs& a,
                                int32_t group, hipStream_t st) {
  return shared_decode_impl(m, a, group, st);
}
hipError_t launch_merge(const AttnArgs& a, hipStream_t st) {
  return merge_impl(a, st);
}
hipError_t launch_generic(const PagedMap& m, const AttnArgs& a, int32_t group,
                          hipStream_t st) {
  return generic_impl(m, a, group, st);
}
hipError_t launch_generic(const ContigMap& m, const AttnArgs& a, int32_t group,
                          hipStream_t st) {
  return generic_impl(m, a, group, st);
}
hipError_t launch_prefill_mfma(const PagedMap& m, const AttnArgs& a,
                               int32_t group, hipStream_t st) {
  return prefill_impl(m, a, group, st);
}
hipError_t launch_prefill_mfma(const ContigMap& m, const AttnArgs& a,
                               int32_t group, hipStream_t st) {
  return prefill_impl(m, a, group, st);
}

}  // namespace pkv
