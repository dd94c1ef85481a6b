// Sparse core attention over the per-row top-k: the consumer of the indexer's
// selection (the v1 listing "SPIN: Shadow Predictive Indexer for Sparse
// Attention", Abstract: a fixed top-k of tokens goes to core attention).
//
// Every one of the 128 query heads of a row attends to one shared cache row
// per selected token (576 bf16 values; the value is its first 512, the
// absorbed form of multi-head latent attention).  One workgroup takes one
// row and one contiguous share of its top-k list, in tiles of 32 tokens;
// wave w owns heads 32w .. 32w + 31.  Per tile:
//   - the 32 cache rows are gathered into LDS twice: row-major (the A
//     operand of S^T = K Q^T) and transposed, with the tokens of each lane's
//     MFMA k-group stored contiguously (the A operand of O^T += V^T P^T);
//   - S^T comes out of 36 v_mfma_f32_32x32x16_bf16 with Q^T held by each
//     lane (28 of its 36 k-steps in registers, 8 in the lane's own LDS
//     slots), so each lane holds 16 scores of one head;
//   - the online softmax (base 2) turns them into bf16 weights that are
//     already in the B-operand layout of the 32 PV MFMAs (registers 8ks..8ks+7
//     are k-step ks), with no shuffle;
//   - O^T accumulates in 16 32x32 tiles per wave (512 channels x 32 heads).
// The cache rows of a share are resolved (top-k entry -> block table -> row)
// once, before the first tile, and each tile's gather is issued into
// registers before the previous tile's MFMAs.  The softmax weights are taken
// against a reference maximum that moves only when a tile passes it by more
// than 2^8, so the rescale of O is rare.  With more than one share per row,
// each share writes its normalised output (bf16) and log-sum-exp, and a second
// kernel merges them in fp32.
#include "spin_attention.h"
#include "spin_device.h"

namespace spin {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAT = 32;                               // tokens per tile
constexpr int kAWaves = kAttnHeads / 32;              // 32 heads per wave
constexpr int kAThreads = kAWaves * kWave;
constexpr int kKRow = kAttnDim + 8;                   // bf16 per row-major row in LDS
constexpr int kVRow = kAT + 8;                        // bf16 per transposed (channel) row
constexpr int kChunks = kAttnDim / 8;                 // 16-byte chunks per cache row
constexpr int kItems = (kAT / 4) * kChunks;           // (token quad, chunk) staging items
constexpr int kItemsPerThread = (kItems + 255) / 256;
constexpr int kQChunks = kAttnDim / 16;               // Q^T operand chunks (k-steps) per lane
constexpr int kQReg = 28;                  // chunks held in registers, the rest in LDS
constexpr int kQLds = kQChunks - kQReg;
constexpr int kMfmaGroup = 6;       // MFMAs between scheduling fences
constexpr int kMaxShare = 4096;                       // top-k entries per share (<= topk)
constexpr int kMaxShares = 16;                        // shares per row at most
constexpr double kMergeCostPerShare = 0.008;          // merge cost of one share-row, in tile-times
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;                  // reference-max slack (base 2)

struct AttnArgs {
  spin_batch bt;
  int K, splits, chunk;
  float scale_log2;                 // scale * log2(e)
  const uint16_t* q;                // [rows][128][576] bf16
  const uint16_t* kv;               // [pool_pages * 64][576] bf16
  int64_t pool_pages;
  const int32_t* table;             // [B][max_blocks]
  const int32_t* topk;              // [rows][K]
  uint16_t* out;                    // [rows][128][512] bf16
  float* lse;                       // [rows][128]
  uint16_t* ws_o;                   // [rows][splits][128][512] bf16, normalised per share
  float* ws_lse;                    // [rows][splits][128]
};

__device__ __forceinline__ bool row_ok(const spin_batch& bt, int b) {
  const int q0 = bt.qpos[b];
  return q0 >= 0 && q0 <= bt.max_blocks * kBlock - bt.R;
}

__device__ __forceinline__ uint32_t half16(const uint4& x, int c) {
  const uint32_t w = c < 2 ? x.x : (c < 4 ? x.y : (c < 6 ? x.z : x.w));
  return (c & 1) ? (w >> 16) : (w & 0xFFFFu);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const __bf16 h = __bf16(f);
  return uint32_t(__builtin_bit_cast(uint16_t, h));
}

// position of tile token t in a transposed row: the 8 tokens that lane group
// h of k-step ks multiplies (16ks + 8a + 4h + r, a, r varying) sit at
// 16ks + 8h .. 16ks + 8h + 7
__device__ __forceinline__ int vt_pos(int t) {
  return 16 * (t >> 4) + 8 * ((t >> 2) & 1) + 4 * ((t >> 3) & 1) + (t & 3);
}

__global__ void __launch_bounds__(kAThreads, 1)
k_attention(AttnArgs a) {
  __shared__ __align__(16) uint16_t s_k[kAT * kKRow];
  __shared__ __align__(16) uint16_t s_vt[kAttnValueDim * kVRow];
  __shared__ int s_tok[kMaxShare];          // pool row of each entry of the share, -1 = skipped
  __shared__ uint32_t s_mask[kMaxShare / kAT];
  __shared__ __align__(16) uint16_t s_q[kAWaves * (kQLds > 0 ? kQLds : 1) * kWave * 8];

  const int split = blockIdx.x, row = blockIdx.y;
  const int b = row / a.bt.R, r = row - b * a.bt.R;
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  const int hg = l >> 5, n = l & 31;
  const int head = 32 * w + n;
  const bool ok = row_ok(a.bt, b);
  const int qr = a.bt.qpos[b] + r;
  const int e0 = split * a.chunk;
  const int e1 = min(a.K, e0 + a.chunk);

  // Q^T operand: chunk c holds dims 16c + 8hg .. 16c + 8hg + 7 of this lane's head.
  // The first kQReg chunks stay in registers; each lane parks the others in
  // its own 16-byte LDS slots.  Without that the kernel spills to scratch, and
  // a scratch reload waits on the same in-order counter as the next tile's
  // gather, which then never overlaps the MFMAs.
  bf16x8 qv[kQReg];
  const uint16_t* qrow = a.q + (size_t(row) * kAttnHeads + head) * kAttnDim;
#pragma unroll
  for (int c = 0; c < kQChunks; ++c) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * hg);
    if (c < kQReg)
      qv[c] = x;
    else
      *reinterpret_cast<bf16x8*>(&s_q[((w * kQLds + c - kQReg) * kWave + l) * 8]) = x;
  }

  f32x16 acc[kAttnValueDim / 32];
#pragma unroll
  for (int ct = 0; ct < kAttnValueDim / 32; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[ct][i] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;

  // the share's cache rows, resolved once: top-k entry -> block table -> row
  const int n_share = ok ? max(0, e1 - e0) : 0;
  for (int i = tid; i < (n_share + kAT - 1) / kAT * kAT; i += kAThreads) {
    int prow = -1;
    if (i < n_share) {
      const int p = a.topk[size_t(row) * a.K + e0 + i];
      if (p >= 0 && p <= qr) {
        const int pg = a.table[size_t(b) * a.bt.max_blocks + p / kBlock];
        if (pg >= 0 && pg < a.pool_pages) prow = pg * kBlock + (p & (kBlock - 1));
      }
    }
    s_tok[i] = prow;
    const uint64_t bal = __ballot(prow >= 0);     // i - l is a multiple of 64
    if (l == 0) {
      s_mask[i / kAT] = uint32_t(bal);
      s_mask[i / kAT + 1] = uint32_t(bal >> 32);
    }
  }
  __syncthreads();

  // Gather of tile t0 into registers: item (token quad tq, 16-byte chunk cc).
  // Items run tq-fastest, so the 16 lanes of a transposed store cover 8 token
  // quads x 2 chunks: 32 distinct banks.  The next tile's loads are issued
  // before the current tile's MFMAs, so their latency overlaps them.
  uint4 gq[kItemsPerThread][4];
  auto issue = [&](int t0) {
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
      const int it = tid + k * kAThreads;
      const int tq = it & 7, cc = it >> 3;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int prow = it < kItems ? s_tok[t0 + 4 * tq + u] : -1;
        gq[k][u] = *reinterpret_cast<const uint4*>(a.kv + size_t(prow < 0 ? 0 : prow) * kAttnDim +
                                                   8 * (it < kItems ? cc : 0));
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int k = 0; k < kItemsPerThread; ++k) {
      const int it = tid + k * kAThreads;
      if (it >= kItems) continue;
      const int tq = it & 7, cc = it >> 3;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<uint4*>(&s_k[(4 * tq + u) * kKRow + 8 * cc]) = gq[k][u];
      if (cc < kAttnValueDim / 8) {
        const int p0 = vt_pos(4 * tq);
#pragma unroll
        for (int c2 = 0; c2 < 8; ++c2) {
          uint2 v;
          v.x = half16(gq[k][0], c2) | (half16(gq[k][1], c2) << 16);
          v.y = half16(gq[k][2], c2) | (half16(gq[k][3], c2) << 16);
          *reinterpret_cast<uint2*>(&s_vt[(8 * cc + c2) * kVRow + p0]) = v;
        }
      }
    }
  };

  // Every load so far (Q, the top-k entries, the block table) is complete
  // before the tile loop, so that no wait inside it on one of them (in-order
  // vmcnt) can also wait for the next tile's gather.
  __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0); expcnt, lgkmcnt unchanged
  if (n_share > 0) issue(0);
  for (int t0 = 0; t0 < n_share; t0 += kAT) {
    const uint32_t vmask = s_mask[t0 / kAT];
    stage();
    __syncthreads();
    if (t0 + kAT < n_share) issue(t0 + kAT);
    if (vmask != 0) {
      f32x16 s;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&s_k[n * kKRow + 16 * c + 8 * hg]);
        const bf16x8 qb =
            c < kQReg ? qv[c < kQReg ? c : 0]
                      : *reinterpret_cast<const bf16x8*>(&s_q[((w * kQLds + c - kQReg) * kWave + l) * 8]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb, s, 0, 0, 0);
        if (c % kMfmaGroup == kMfmaGroup - 1) __builtin_amdgcn_sched_barrier(0);   // bound the reads in flight
      }

      // online softmax in base 2; register i holds token 8(i/4) + 4hg + i%4
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = 8 * (i >> 2) + 4 * hg + (i & 3);
        x[i] = ((vmask >> tok) & 1u) ? s[i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      // The weights are taken against a reference m that moves only when the
      // tile's maximum passes it by more than kRescaleLog2: weights stay below
      // 2^kRescaleLog2, o and l share the reference, and o / l is unchanged,
      // while the 256-register rescale of o runs on few tiles.
      const float mnew = (mx > m + kRescaleLog2) ? mx : m;   // m = -inf: the first tile moves it
      const float alpha = exp2f(m - mnew);         // 0 on the first tile, 1 unless m moved
      float psum = 0.0f;
      bf16x8 pb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(x[i] - mnew);
        psum += p;
        pb[i >> 3][i & 7] = __bf16(p);
      }
      lsum = lsum * alpha + psum;
      m = mnew;
      if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
        for (int ct = 0; ct < kAttnValueDim / 32; ++ct)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[ct][i] *= alpha;
      }
#pragma unroll
      for (int ct = 0; ct < kAttnValueDim / 32; ++ct)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 va =
              *reinterpret_cast<const bf16x8*>(&s_vt[(32 * ct + n) * kVRow + 16 * ks + 8 * hg]);
          acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], acc[ct], 0, 0, 0);
          if ((2 * ct + ks) % kMfmaGroup == kMfmaGroup - 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();              // the next tile overwrites s_k and s_vt
  }

  // lane pair (l, l ^ 32) covers the head's 32 tokens per tile
  const float ltot = lsum + __shfl_xor(lsum, 32, kWave);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  const float lse = !ok ? __builtin_nanf("") : (ltot > 0.0f ? (m + log2f(ltot)) * kLn2 : -INFINITY);
  // register i of tile ct holds channel 32ct + 8(i/4) + 4hg + i%4
  if (a.splits == 1) {
    uint16_t* o = a.out + (size_t(row) * kAttnHeads + head) * kAttnValueDim;
#pragma unroll
    for (int ct = 0; ct < kAttnValueDim / 32; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v;
        v.x = bf16_bits(acc[ct][4 * g] * inv) | (bf16_bits(acc[ct][4 * g + 1] * inv) << 16);
        v.y = bf16_bits(acc[ct][4 * g + 2] * inv) | (bf16_bits(acc[ct][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(o + 32 * ct + 8 * g + 4 * hg) = v;
      }
    if (hg == 0) a.lse[size_t(row) * kAttnHeads + head] = lse;
  } else {
    const size_t part = (size_t(row) * a.splits + split) * kAttnHeads + head;
    uint16_t* o = a.ws_o + part * kAttnValueDim;
#pragma unroll
    for (int ct = 0; ct < kAttnValueDim / 32; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v;
        v.x = bf16_bits(acc[ct][4 * g] * inv) | (bf16_bits(acc[ct][4 * g + 1] * inv) << 16);
        v.y = bf16_bits(acc[ct][4 * g + 2] * inv) | (bf16_bits(acc[ct][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(o + 32 * ct + 8 * g + 4 * hg) = v;
      }
    if (hg == 0) a.ws_lse[part] = lse;
  }
}

constexpr int kCombineGroups = 64;                    // head groups per row in the merge (one item per thread)

// Merge of the shares of each row: lse = log sum_s exp(lse_s),
// o = sum_s exp(lse_s - lse) o_s.  grid (rows, kCombineGroups), 256 threads;
// thread item (head, 4-channel group).
__global__ void __launch_bounds__(256)
k_attention_combine(AttnArgs a) {
  const int row = blockIdx.x;
  const int b = row / a.bt.R;
  const bool ok = row_ok(a.bt, b);
  constexpr int kHeadsPerGroup = kAttnHeads / kCombineGroups;
  for (int it = threadIdx.x; it < kHeadsPerGroup * (kAttnValueDim / 4); it += 256) {
    const int head = blockIdx.y * kHeadsPerGroup + it / (kAttnValueDim / 4);
    const int cq = it % (kAttnValueDim / 4);
    const size_t base = size_t(row) * a.splits * kAttnHeads + head;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.ws_lse[base + size_t(s) * kAttnHeads]);
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float den = 0.0f;
    if (ok && mx > -INFINITY) {
      for (int s = 0; s < a.splits; ++s) {
        const size_t part = base + size_t(s) * kAttnHeads;
        const float wgt = __expf(a.ws_lse[part] - mx);
        const uint2 v = *reinterpret_cast<const uint2*>(a.ws_o + part * kAttnValueDim + 4 * cq);
        den += wgt;
        o.x += wgt * __uint_as_float(v.x << 16);
        o.y += wgt * __uint_as_float(v.x & 0xFFFF0000u);
        o.z += wgt * __uint_as_float(v.y << 16);
        o.w += wgt * __uint_as_float(v.y & 0xFFFF0000u);
      }
      const float inv = 1.0f / den;
      o.x *= inv;
      o.y *= inv;
      o.z *= inv;
      o.w *= inv;
    }
    uint2 v;
    v.x = bf16_bits(o.x) | (bf16_bits(o.y) << 16);
    v.y = bf16_bits(o.z) | (bf16_bits(o.w) << 16);
    *reinterpret_cast<uint2*>(a.out + (size_t(row) * kAttnHeads + head) * kAttnValueDim + 4 * cq) = v;
    if (cq == 0)
      a.lse[size_t(row) * kAttnHeads + head] =
          !ok ? __builtin_nanf("") : (mx > -INFINITY ? mx + __logf(den) : -INFINITY);
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

AttnPlan attention_plan(const spin_batch& bt, int topk) {
  AttnPlan p;
  p.rows = bt.B * bt.R;
  const int tiles = (topk + kAT - 1) / kAT;
  // One workgroup fills a CU, so the launch runs in ceil(groups / CUs) rounds
  // of `tiles per share` tiles each; every share adds a partial that the merge
  // reads (about kMergeCostPerShare tile-times per row and share, measured).
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  int best = 1;
  double best_cost = 0.0;
  for (int sp = 1; sp <= kMaxShares && sp <= tiles; ++sp) {
    const double rounds = double((int64_t(p.rows) * sp + cus - 1) / cus);
    const double cost = rounds * double((tiles + sp - 1) / sp) +
                        (sp > 1 ? kMergeCostPerShare * p.rows * sp : 0.0);
    if (sp == 1 || cost < best_cost) {
      best = sp;
      best_cost = cost;
    }
  }
  p.chunk = ((tiles + best - 1) / best) * kAT;
  p.splits = (topk + p.chunk - 1) / p.chunk;
  p.ws_o_bytes = p.splits > 1 ? align256(size_t(p.rows) * p.splits * kAttnHeads * kAttnValueDim * 2)
                              : 0;
  p.ws_bytes = p.splits > 1 ? p.ws_o_bytes + align256(size_t(p.rows) * p.splits * kAttnHeads * 4)
                            : 0;
  return p;
}

hipError_t launch_attention(const spin_batch& bt, int topk, const int32_t* topk_idx,
                            const void* q, const void* kv, int64_t pool_pages,
                            const int32_t* table, float scale, void* out, float* lse,
                            void* ws, hipStream_t s) {
  const AttnPlan p = attention_plan(bt, topk);
  AttnArgs a;
  a.bt = bt;
  a.K = topk;
  a.splits = p.splits;
  a.chunk = p.chunk;
  a.scale_log2 = scale * 1.44269504088896340736f;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv);
  a.pool_pages = pool_pages;
  a.table = table;
  a.topk = topk_idx;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.ws_o = p.splits > 1 ? static_cast<uint16_t*>(ws) : nullptr;
  a.ws_lse = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_o_bytes) : nullptr;
  hipLaunchKernelGGL(k_attention, dim3(p.splits, p.rows), dim3(kAThreads), 0, s, a);
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attention_combine, dim3(p.rows, kCombineGroups), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace spin
