// Block-sparse ragged causal prefill on matrix cores.
//
// [FI] vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer,
//      MiniMaxM3SparseFlashInferImpl.forward (msa_sparse_attention: ragged
//      rows by cu_seqlens_q, causal, per-token top-k blocks).
// [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4,
//      MiniMaxM3SparseRocmNvfp4Impl / MetadataBuilder.build (each prefill
//      token's request and absolute position).
// [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa,
//      _write_sparse_block_table_row_from_values (the tokens a row sees).
//
// Work decomposition.  A workgroup (4 waves) owns one kv head and QT
// consecutive query rows of one request (QT = 24 for 8 query heads per kv
// head, 12 for 16).  Every query row picks its own blocks, so the workgroup
// first builds, per block of the request, the bit mask of its rows that
// selected it (and may see it causally), then walks the blocks some row
// selected in ascending order.  Each such block's K and V (128 keys x 256 B)
// go once into LDS, double-buffered.  K is copied by direct global-to-LDS
// loads as [key][d] with 16-byte chunks XOR-swizzled by key (each lane's LDS
// slot is fixed, so the swizzle is made by choosing which global chunk the
// lane fetches).  V is loaded into registers, transposed there (8 keys x 8
// d per thread) and stored as V^T [32-key chunk][d][keys], keys in the order
// the P operand holds them, chunks swizzled by d.  Both operands are then
// plain 16-byte LDS reads.  Every wave
// owns 3 matrix tiles of 16 rows = (16 / G query rows) x (G heads) and runs
// QK^T and PV only for the tiles whose rows selected the block; the other
// rows of an active tile are masked.  Online softmax state stays in
// registers; the workgroup writes its rows' bf16 outputs at the end.
// Workgroups of one kv head share an XCD (blockIdx % Hkv), so K/V blocks
// re-read by neighbouring query tiles hit that XCD's L2.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

constexpr int kPfWaves = 4;
constexpr int kPfTiles = 3;                 // matrix tiles per wave
constexpr int kPfMaxBlocks = 2048;          // request blocks a workgroup can index
constexpr int kPfBlockBytes = kBlockTokens * 256;   // one block of K (or V), bf16, head_dim 128

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// K row swizzle: 16-byte chunk c of key row k sits at chunk c ^ (k & 15).
__device__ __forceinline__ int k_swz(int key) { return key & 15; }

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// K of block `phys` (logical block `blk`), kv head kvh, into LDS kb: 8 direct
// 16-byte loads per lane.  Keys at or past seq_len are read from key 0 of the
// block instead (finite data that gets probability zero), so no NaN of an
// unwritten slot reaches the products.
__device__ __forceinline__ void pf_issue_k(lds_u8* kb, const AttendArgs& a, int kvh, int phys, int blk,
                                           int seq_len) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pg = (int64_t)phys * a.block_page_stride;
  const int64_t head_off = (int64_t)kvh * kPageTokens * 256;
  const int nkeys = seq_len - blk * kBlockTokens;     // keys of this block that exist (>= 1)
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int P = (wave * 8 + s) * 1024 + lane * 16;  // LDS byte this lane fills
    const int key = P >> 8, pc = (P >> 4) & 15;
    const int src = key < nkeys ? key : 0;
    const uint8_t* kp = a.k_base + (pg + (src >> 4)) * a.page_stride + head_off + (src & 15) * 256 +
                        ((pc ^ k_swz(key)) << 4);
    __builtin_amdgcn_global_load_lds(kp, kb + (wave * 8 + s) * 1024, 16, 0, 0);
  }
}

// V of a block into registers: thread (c, g, m) loads keys tau(8g .. 8g+7)
// of 32-key chunk c (4g..4g+3 and 16+4g..16+4g+3), d = 8m .. 8m+7.
__device__ __forceinline__ void pf_load_v(u32x4 (&v)[8], const AttendArgs& a, int kvh, int phys, int blk,
                                          int seq_len) {
  const int tid = threadIdx.x, c = tid >> 6, g = (tid >> 4) & 3, m = tid & 15;
  const int64_t pg = (int64_t)phys * a.block_page_stride + a.v_page_offset;
  const int64_t head_off = (int64_t)kvh * kPageTokens * 256;
  const int nkeys = seq_len - blk * kBlockTokens;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = c * 32 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
    const int src = key < nkeys ? key : 0;
    v[i] = *reinterpret_cast<const u32x4*>(a.v_base + (pg + (src >> 4)) * a.page_stride + head_off +
                                           (src & 15) * 256 + m * 16);
  }
}

// Transpose the thread's 8 keys x 8 d and store V^T rows d = 8m + e.
__device__ __forceinline__ void pf_store_vt(const u32x4 (&v)[8], uint8_t* vt_base) {
  const int tid = threadIdx.x, c = tid >> 6, g = (tid >> 4) & 3, m = tid & 15;
  uint8_t* vt = vt_base + c * 128 * 64;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a0 = v[2 * p][e >> 1], a1 = v[2 * p + 1][e >> 1];
      o[p] = (e & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
    }
    const int d = 8 * m + e;
    *reinterpret_cast<u32x4*>(&vt[d * 64 + ((g ^ ((d >> 2) & 3)) << 4)]) = o;
  }
}

struct PfWave {
  static constexpr int KK = 4, NN = 8;
  bf16x8 qop[kPfTiles][KK];
  f32x4 acc[kPfTiles][NN];
  float m[kPfTiles], l[kPfTiles];
  int lrow[kPfTiles];     // row within the workgroup tile, or -1
  int lpos[kPfTiles];     // that row's absolute position
};

// One selected block against this wave's tiles.
__device__ __forceinline__ void pf_compute_block(PfWave& w, const uint8_t* kb, const uint8_t* vtb, uint32_t bmask,
                                                 int blk, int wave, int RT, float sl2) {
  constexpr int KK = PfWave::KK, NN = PfWave::NN;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int kpos_blk = blk * kBlockTokens;
  for (int c = 0; c < 4; ++c) {
    // operands of this 32-key chunk, shared by the wave's active tiles
    bf16x8 kop[2][KK];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int key = c * 32 + 16 * tt + r;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kop[tt][kk] = *reinterpret_cast<const bf16x8*>(kb + key * 256 + (((4 * kk + g) ^ k_swz(key)) << 4));
    }
    // V^T operand of output tile nn: lane (r, g) reads d = 16 nn + r, keys
    // tau(8g .. 8g+7) of the chunk: one 16-byte chunk of the V^T row.
    bf16x8 vop[NN];
    const uint8_t* vt = vtb + c * 128 * 64;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int d = 16 * nn + r;
      vop[nn] = *reinterpret_cast<const bf16x8*>(&vt[d * 64 + ((g ^ ((d >> 2) & 3)) << 4)]);
    }
    const int kbase = kpos_blk + c * 32 + 4 * g;
#pragma unroll
    for (int i = 0; i < kPfTiles; ++i) {
      const uint32_t tile_bits = ((1u << RT) - 1u) << ((wave * kPfTiles + i) * RT);
      if (!(bmask & tile_bits)) continue;
      const bool sel = w.lrow[i] >= 0 && ((bmask >> w.lrow[i]) & 1u);
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s0 = mfma16(kop[0][kk], w.qop[i][kk], s0);
        s1 = mfma16(kop[1][kk], w.qop[i][kk], s1);
      }
      float sc[8];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        sc[ii] = (sel && kbase + ii <= w.lpos[i]) ? s0[ii] * sl2 : -INFINITY;
        sc[4 + ii] = (sel && kbase + 16 + ii <= w.lpos[i]) ? s1[ii] * sl2 : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int ii = 1; ii < 8; ++ii) mx = fmaxf(mx, sc[ii]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(w.m[i], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2_fast(w.m[i] - m_use);
      float p[8], ps = 0.f;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        p[ii] = exp2_fast(sc[ii] - m_use);
        ps += p[ii];
      }
      w.l[i] = w.l[i] * alpha + ps;
      w.m[i] = m_new;
      const u32x4 pw = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        w.acc[i][nn] = w.acc[i][nn] * alpha;
        w.acc[i][nn] = mfma16(vop[nn], pop, w.acc[i][nn]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void prefill_blocks_kernel(const AttendArgs a, int n_slots) {
  constexpr int D = 128, KK = PfWave::KK, NN = PfWave::NN;
  // two K/V buffers as distinct LDS objects: the loop below is unrolled by two,
  // so the compiler knows the in-flight copies target the other buffer
  __shared__ __align__(16) uint8_t k0[kPfBlockBytes], k1[kPfBlockBytes];
  __shared__ __align__(16) uint8_t vt0[kPfBlockBytes], vt1[kPfBlockBytes];
  __shared__ uint32_t s_mask[kPfMaxBlocks];
  __shared__ uint16_t s_list[kPfMaxBlocks];   // selected blocks, ascending
  __shared__ int32_t s_phys[kPfMaxBlocks];    // their physical block ids
  __shared__ int s_info[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int G = a.group, RT = 16 / G, QT = kPfWaves * kPfTiles * RT;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int t = n_slots - 1 - (int)(blockIdx.x / a.num_kv_heads);   // heavy (late) tiles first
  const int R = a.num_reqs;

  // ---- which rows: a tile of one request, padding rows, or nothing
  if (wave == 0) {
    int running = 0, found_req = -1, found_row0 = 0;
    for (int base = 0; base < R; base += 64) {
      const int rq = base + lane;
      const int n = rq < R ? (a.cu_seqlens_q[rq + 1] - a.cu_seqlens_q[rq] + QT - 1) / QT : 0;
      const int incl = wave_incl_scan(n, lane);
      const int excl = incl - n;
      const bool hit = rq < R && t >= running + excl && t < running + incl;
      const uint64_t hm = __ballot(hit);
      if (hm) {
        const int src = __ffsll((unsigned long long)hm) - 1;
        found_req = __shfl(rq, src);
        found_row0 = __shfl(rq < R ? a.cu_seqlens_q[rq] + (t - running - excl) * QT : 0, src);
      }
      running += __shfl(incl, 63);
    }
    if (lane == 0) {
      const int real_end = a.cu_seqlens_q[R];
      if (found_req >= 0) {
        s_info[0] = 0;
        s_info[1] = found_req;
        s_info[2] = found_row0;
        s_info[3] = min(found_row0 + QT, a.cu_seqlens_q[found_req + 1]);
      } else {
        const int p = t - running;   // padding tiles follow the real ones
        s_info[0] = 1;
        s_info[1] = 0;
        s_info[2] = real_end + p * QT;
        s_info[3] = min(real_end + (p + 1) * QT, a.total_rows);
      }
    }
  }
  __syncthreads();
  const int mode = s_info[0], req = s_info[1], row0 = s_info[2], row_end = s_info[3];
  if (row0 >= row_end) return;   // uniform: nothing to do
  if (mode == 1) {
    // padding rows attend nothing: zero their heads of this kv head
    const int per_row = G * D / 8;   // 16-byte stores
    for (int idx = tid; idx < (row_end - row0) * per_row; idx += 256) {
      const int rr = idx / per_row, wd = idx % per_row;
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.out) +
                     (((int64_t)(row0 + rr) * a.num_q_heads + kvh * G) * D) * 2 + wd * 16;
      *reinterpret_cast<u32x4*>(dst) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const int cu0 = a.cu_seqlens_q[req], cu1 = a.cu_seqlens_q[req + 1];
  const int seq_len = a.seq_lens[req];
  const int ctx0 = seq_len - (cu1 - cu0);          // context before the new tokens
  const int pos_first = ctx0 + (row0 - cu0);
  const int pos_last = ctx0 + (row_end - 1 - cu0);
  const int nblk = pos_last < 0 ? 0 : min(pos_last / kBlockTokens + 1, a.bt_cols);
  const int32_t* bt_row = a.block_table + (int64_t)req * a.bt_stride;

  // ---- per-block masks of the rows that selected the block (and may see it)
  for (int j = tid; j < nblk; j += 256) s_mask[j] = 0u;
  __syncthreads();
  const int nrows = row_end - row0;
  for (int idx = tid; idx < nrows * a.topk_k; idx += 256) {
    const int rr = idx / a.topk_k, tk = idx - rr * a.topk_k;
    const int pos = pos_first + rr;
    const int blk = a.topk[(int64_t)(row0 + rr) * a.topk_stride + tk];
    if (pos >= 0 && blk >= 0 && blk <= pos / kBlockTokens && blk < nblk) atomicOr(&s_mask[blk], 1u << rr);
  }
  __syncthreads();
  // ---- selected blocks, ascending (blocks whose pages lie outside the cache are skipped)
  if (wave == 0) {
    int n = 0;
    for (int base = 0; base < nblk; base += 64) {
      const int j = base + lane;
      bool act = j < nblk && s_mask[j] != 0u;
      if (act) {
        const int phys = bt_row[j];
        const int64_t last = (int64_t)phys * a.block_page_stride + a.v_page_offset + kPagesPerBlock - 1;
        act = phys >= 0 && last < a.num_pages;
      }
      const uint64_t am = __ballot(act);
      const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(am >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)am, 0u));
      if (act) {
        s_list[n + rank] = (uint16_t)j;
        s_phys[n + rank] = bt_row[j];
      }
      n += __popcll(am);
    }
    if (lane == 0) s_info[0] = n;
  }

  // ---- this wave's query operands and row data
  PfWave w;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    const int rr = (wave * kPfTiles + i) * RT + r / G;
    const bool ok = r < RT * G && rr < nrows;
    w.lrow[i] = ok ? rr : -1;
    w.lpos[i] = pos_first + rr;
    w.m[i] = -INFINITY;
    w.l[i] = 0.f;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                          (((int64_t)(row0 + (ok ? rr : 0)) * a.num_q_heads + kvh * G + (r % G)) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 q4 = ok ? *reinterpret_cast<const u32x4*>(qrow + 2 * (32 * kk + 8 * g)) : u32x4{0u, 0u, 0u, 0u};
      w.qop[i][kk] = __builtin_bit_cast(bf16x8, q4);
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) w.acc[i][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float kscale = a.k_scale ? *a.k_scale : 1.f;
  const float sl2 = a.softmax_scale * kscale * kLog2e;
  __syncthreads();
  const int n_act = s_info[0];

  u32x4 vst[8];
  if (n_act > 0) {
    const int j = s_list[0];
    pf_load_v(vst, a, kvh, s_phys[0], j, seq_len);
    pf_issue_k((lds_u8*)k0, a, kvh, s_phys[0], j, seq_len);
    pf_store_vt(vst, vt0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t wave_bits = ((1u << (kPfTiles * RT)) - 1u) << (wave * kPfTiles * RT);
  for (int it = 0; it < n_act; it += 2) {
    // even step: compute from buffer 0 while buffer 1 fills
    {
      const int j = s_list[it];
      const bool more = it + 1 < n_act;
      if (more) {
        const int jn = s_list[it + 1], pn = s_phys[it + 1];
        pf_load_v(vst, a, kvh, pn, jn, seq_len);
        pf_issue_k((lds_u8*)k1, a, kvh, pn, jn, seq_len);
      }
      const uint32_t bmask = s_mask[j];
      if (bmask & wave_bits) pf_compute_block(w, k0, vt0, bmask, j, wave, RT, sl2);
      if (more) pf_store_vt(vst, vt1);
      __builtin_amdgcn_s_waitcnt(0);   // this lane's copies of the next block have landed
      __syncthreads();
    }
    if (it + 1 >= n_act) break;
    // odd step: compute from buffer 1 while buffer 0 fills
    {
      const int j = s_list[it + 1];
      const bool more = it + 2 < n_act;
      if (more) {
        const int jn = s_list[it + 2], pn = s_phys[it + 2];
        pf_load_v(vst, a, kvh, pn, jn, seq_len);
        pf_issue_k((lds_u8*)k0, a, kvh, pn, jn, seq_len);
      }
      const uint32_t bmask = s_mask[j];
      if (bmask & wave_bits) pf_compute_block(w, k1, vt1, bmask, j, wave, RT, sl2);
      if (more) pf_store_vt(vst, vt0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- outputs: lane holds head r % G of row lrow, d = 16 nn + 4 g + ii
  const float vscale = a.v_scale ? *a.v_scale : 1.f;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    float L = w.l[i];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    if (w.lrow[i] < 0) continue;
    const float inv = L > 0.f ? vscale / L : 0.f;
    uint8_t* orow = reinterpret_cast<uint8_t*>(a.out) +
                    (((int64_t)(row0 + w.lrow[i]) * a.num_q_heads + kvh * G + (r % G)) * D) * 2;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int d = 16 * nn + 4 * g;
      const u32x2 o = {pack_bf16(w.acc[i][nn][0] * inv, w.acc[i][nn][1] * inv),
                       pack_bf16(w.acc[i][nn][2] * inv, w.acc[i][nn][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d * 2) = o;
    }
  }
}

hipError_t launch_prefill_blocks(const AttendArgs& a, hipStream_t stream) {
  const int QT = kPfWaves * kPfTiles * (16 / a.group);
  const int n_slots = (a.total_rows + QT - 1) / QT + a.num_reqs + 1;
  const int64_t blocks = (int64_t)n_slots * a.num_kv_heads;
  hipLaunchKernelGGL(prefill_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n_slots);
  return hipGetLastError();
}

bool prefill_blocks_supported(int group, int head_dim, int fmt, int bt_cols) {
  return (group == 8 || group == 16) && head_dim == 128 && fmt == kFmtBf16 && bt_cols <= kPfMaxBlocks;
}

}  // namespace msa
