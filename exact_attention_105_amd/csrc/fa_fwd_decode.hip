// Attention forward for few query rows per head (decode), bfloat16, gfx950.
//
// With Nq small the work is a stream over K and V (page "FlashAttention 4",
// centron.de, on why attention stays memory-bound: every query token reads
// thousands of keys and their values).  This kernel is built for that
// stream:
//   * grouped-query packing: the Nq x G query rows that read one key/value
//     head (G = Hq / Hkv; page "Flash Attention", 21medien.de, key techniques:
//     multi-query / grouped-query attention) share one 32-column MFMA block,
//     so K and V of a head are read once, not G times;
//   * one workgroup per (batch, key/value head, 32 packed rows); its four
//     waves split the keys into four contiguous ranges and stream them
//     independently, each through its own double-buffered LDS region filled
//     by direct global->LDS copies, so the key loop has no barriers;
//   * each wave runs the same online softmax as the prefill kernels over its
//     range; the four partial results (running max, sum, unnormalised O) are
//     merged at the end through LDS with the same rescaling rule (the merge
//     step of page "FlashAttention (DE)", systems-analysis.info, section
//     "Online-Softmax-Berechnung", applied across ranges instead of tiles).
// Split-KV: with few (batch, key/value head) units the grid cannot fill the
// GPU, so the keys can also be split over n_splits workgroups.  Each then
// writes its normalised fp32 partial O and its base-2 LSE to the caller's
// workspace, and fa_decode_merge_kernel combines the splits with the same
// rescaling rule (O = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M)).
// Packed row r of row tile rt is query index i = (32*rt + r) / G of query
// head hkv*G + (32*rt + r) % G.  Products, masking, softmax and LDS layouts
// follow fa_fwd_bf16.hip (S^T = K Q^T, O^T += V^T P^T, transposing V reads).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr float kDecRescaleLog2 = 8.0f;
constexpr int kD = 128;
constexpr int kNW = 4;                 // waves, each owning a quarter of the keys
constexpr int kBN = 32;                // keys per tile
constexpr int kROW = kD * 2;           // bytes per K/V row
constexpr int kTILE = kBN * kROW;      // 8 KiB
constexpr int kWSTAGE = 2 * kTILE;     // K + V of one tile
constexpr int kWLDS = 2 * kWSTAGE;     // two stages per wave: 32 KiB
constexpr int kLDS = kNW * kWLDS;      // 128 KiB
constexpr int kCH = kTILE / 1024;      // 1 KiB copies per tile and tensor: 8

}  // namespace

__global__ __launch_bounds__(256, 1) void fa_fwd_decode_kernel(FwdParams p, int causal, int n_splits, float* ws) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[kLDS];
    lds_char* smem = (lds_char*)smem_raw;
    const uint32_t smem_u32 = (uint32_t)(uintptr_t)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int g = lane >> 5;

    // workgroup -> (key split, row tile, batch, key/value head)
    const int units = p.B * p.Hkv;
    const int unit = blockIdx.x % units;
    const int row_tiles = (p.Nq * p.group + 31) / 32;
    const int tsel = blockIdx.x / units;
    const int rt = tsel % row_tiles;
    const int split = tsel / row_tiles;
    const int b = unit / p.Hkv;
    const int hkv = unit % p.Hkv;
    const int G = p.group;
    const int packed = p.Nq * G;                 // packed rows of this (b, hkv)
    const int r = 32 * rt + n;                   // this lane's packed row
    const bool row_ok = r < packed;
    const int qi = row_ok ? r / G : 0;           // query index
    const int hq = hkv * G + (row_ok ? r % G : 0);

    const char* Kh = reinterpret_cast<const char*>(p.k) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * kROW;
    const char* Vh = reinterpret_cast<const char*>(p.v) + ((int64_t)(b * p.Hkv + hkv) * p.Nk) * kROW;

    // Q row of this lane (packed row r) as the B operand.
    bf16x8 qf[kD / 16];
    if (row_ok) {
        const char* src = reinterpret_cast<const char*>(p.q) + (((int64_t)(b * p.Hq + hq) * p.Nq + qi) * kD) * 2;
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
            u32x4 x = ldg16(src + (2 * ks + g) * 16);
            x ^= p.q_sign;
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
    // last visible key of this row (bottom-right causal), else the last key
    const int lim_row = (causal && row_ok) ? min(qi + p.causal_shift, p.Nk - 1) : p.Nk - 1;

    // this workgroup's key split and this wave's quarter of it, in whole tiles
    const int n_tiles_all = (p.Nk + kBN - 1) / kBN;
    const int per_split = (n_tiles_all + n_splits - 1) / n_splits;
    const int s0 = min(split * per_split, n_tiles_all);
    const int s1 = min(s0 + per_split, n_tiles_all);
    const int per = (s1 - s0 + kNW - 1) / kNW;
    const int t0 = min(s0 + w * per, s1);
    const int t1 = min(t0 + per, s1);

    // per-lane copy offsets: chunk c holds tile rows 4c .. 4c+3
    const int c_row = lane >> 4, c_su = lane & 15;
    uint32_t dk_off[kCH], dv_off[kCH];
#pragma unroll
    for (int c = 0; c < kCH; ++c) {
        const int row = 4 * c + c_row;
        dk_off[c] = row * kROW + ((c_su ^ (row & 15)) << 4);
        dv_off[c] = row * kROW + ((c_su ^ (4 * (row & 3))) << 4);
    }
    uint32_t k_off[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) k_off[ks] = n * kROW + (((2 * ks + g) ^ (n & 15)) << 4);
    // V rows are swizzled by 4*(row mod 4) units: the 4 rows x 64 bytes of one
    // transposing-read cycle then cover all 64 banks.
    uint32_t v_off[kD / 32];
    {
        const int tr_row = 4 * g + ((n & 15) >> 2);
        const int tr_d = 16 * (n >> 4) + 4 * (n & 3);
#pragma unroll
        for (int db = 0; db < kD / 32; ++db) {
            const int d = 32 * db + tr_d;
            v_off[db] = tr_row * kROW + (((d >> 3) ^ (4 * (tr_row & 3))) << 4) + (d & 7) * 2;
        }
    }

    const uint32_t wbase = smem_u32 + w * kWLDS;
    auto issue_tile = [&](int j, int stage) {
        const uint32_t kdst = wbase + stage * kWSTAGE;
        const uint32_t vdst = kdst + kTILE;
        const int key0 = j * kBN;
        const char* kb = Kh + (int64_t)key0 * kROW;
        const char* vb = Vh + (int64_t)key0 * kROW;
        if (key0 + kBN <= p.Nk) {
#pragma unroll
            for (int c = 0; c < kCH; ++c) {
                dma16(kb, dk_off[c], kdst + c * 1024);
                dma16(vb, dv_off[c], vdst + c * 1024);
            }
        } else {
#pragma unroll
            for (int c = 0; c < kCH; ++c) {
                const int row = 4 * c + c_row;
                const int rc = copy_src_row(row, key0, p.Nk);
                dma16(kb, rc * kROW + ((c_su ^ (row & 15)) << 4), kdst + c * 1024);
                dma16(vb, rc * kROW + ((c_su ^ (4 * (row & 3))) << 4), vdst + c * 1024);
            }
        }
    };

    f32x16 o[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) o[db] = f32x16{};
    float mref = -INFINITY;
    float l = 0.f;

    if (t0 < t1) issue_tile(t0, 0);
    for (int j = t0; j < t1; ++j) {
        const int stage = (j - t0) & 1;
        FA_WAIT_VMCNT(0);                       // this wave's copies of tile j landed
        __builtin_amdgcn_wave_barrier();
        if (j + 1 < t1) issue_tile(j + 1, stage ^ 1);
        const lds_char* kb = smem + w * kWLDS + stage * kWSTAGE;
        const lds_char* vb = kb + kTILE;
        const int key0 = j * kBN;

        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) s = mfma_bf16_32x32x16(lds_b128(kb + k_off[ks]), qf[ks], s);

        if (key0 + kBN - 1 > lim_row || !row_ok) {
            const int lim = lim_row - key0 - 4 * g;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (8 * (i >> 2) + (i & 3) > lim) s[i] = -INFINITY;
        }

        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        mx = pair_max(mx) * p.c;
        const bool move = mx > mref + kDecRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float mnew = move ? mx : mref;
            const float alpha = move ? ((mref == -INFINITY) ? 0.f : fast_exp2(mref - mnew)) : 1.f;
            mref = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < kD / 32; ++db) o[db] *= alpha;
        }
        const float mb = (mref == -INFINITY) ? 0.f : mref;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = fast_exp2(fmaf(s[i], p.c, -mb));
            s[i] = e;
            rs += e;
        }
        l += rs;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            u32x4 pk;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) pk[e2] = pack_bf16x2(s[8 * h8 + 2 * e2], s[8 * h8 + 2 * e2 + 1]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
            for (int db = 0; db < kD / 32; ++db) {
                const lds_char* vp = vb + v_off[db] + 16 * h8 * kROW;
                const i16x4 lo = lds_tr16(vp);
                const i16x4 hi = lds_tr16(vp + 8 * kROW);
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = mfma_bf16_32x32x16(a, pb, o[db]);
            }
        }
    }

    // Merge the four key ranges.  LDS: per wave 32 rows x 128 d fp32 (16 KiB)
    // followed by the per-row (reference, sum) pairs.
    const float lt = pair_sum(l);
    __syncthreads();                            // every wave is done with its copies
    float* part = reinterpret_cast<float*>(smem_raw);           // [NW][32][128]
    float* stat = part + kNW * 32 * kD;                           // [NW][32][2]
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = 32 * db + 8 * i4 + 4 * g;
            *reinterpret_cast<f32x4*>(part + (w * 32 + n) * kD + d) =
                f32x4{o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]};
        }
    if (g == 0) {
        stat[(w * 32 + n) * 2 + 0] = mref;
        stat[(w * 32 + n) * 2 + 1] = lt;
    }
    __syncthreads();
    {
        const int row = tid >> 3;               // packed row 0..31
        const int d0 = (tid & 7) * 16;          // 16 output columns per thread
        const int rr = 32 * rt + row;
        if (rr < packed) {
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, stat[(ww * 32 + row) * 2]);
            float L = 0.f;
            float acc[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int ww = 0; ww < kNW; ++ww) {
                    const float mw = stat[(ww * 32 + row) * 2];
                    const float a = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
                    L += a * stat[(ww * 32 + row) * 2 + 1];
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[e] += a * part[(ww * 32 + row) * kD + d0 + e];
                }
            }
            const float inv = L > 0.f ? p.o_scale / L : 0.f;
            const int i = rr / G, h = hkv * G + rr % G;
            const int64_t orow_idx = (int64_t)(b * p.Hq + h) * p.Nq + i;
            if (n_splits == 1) {
                char* orow = reinterpret_cast<char*>(p.o) + (orow_idx * kD + d0) * 2;
                u32x4 v0, v1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v0[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
                    v1[e] = pack_bf16x2(acc[8 + 2 * e] * inv, acc[8 + 2 * e + 1] * inv);
                }
                *reinterpret_cast<u32x4*>(orow) = v0;
                *reinterpret_cast<u32x4*>(orow + 16) = v1;
                if (p.lse != nullptr && (tid & 7) == 0)
                    p.lse[orow_idx] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
            } else {
                // this split's partial: normalised fp32 O, and its base-2 LSE
                const int64_t R = (int64_t)p.B * p.Hq * p.Nq;
                float* op = ws + ((int64_t)split * R + orow_idx) * kD + d0;
#pragma unroll
                for (int e = 0; e < 16; e += 4)
                    *reinterpret_cast<f32x4*>(op + e) =
                        f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
                if ((tid & 7) == 0)
                    ws[(int64_t)n_splits * R * kD + (int64_t)split * R + orow_idx] =
                        L > 0.f ? M + __builtin_amdgcn_logf(L) : -INFINITY;
            }
        }
    }
}

// Combine the n_splits partials of one output row (one workgroup per row,
// one thread per column of d): weights 2^(lse_s - M), M the largest lse_s.
// The split LSEs are read in parallel (thread s reads splits s and s + kD),
// the maximum and the sum of the weights are reduced across the two waves,
// the weights go to LDS, and each thread then sums its column over the
// splits with several loads in flight.
__global__ __launch_bounds__(kD) void fa_decode_merge_kernel(FwdParams p, int n_splits, const float* ws) {
    __shared__ float wgt[2 * kD];
    __shared__ float red[2][kD / 64];
    const int64_t R = (int64_t)p.B * p.Hq * p.Nq;
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const int wv = t >> 6;
    const float* lse2 = ws + (int64_t)n_splits * R * kD;
    const float l0 = t < n_splits ? lse2[(int64_t)t * R + r] : -INFINITY;
    const float l1 = t + kD < n_splits ? lse2[(int64_t)(t + kD) * R + r] : -INFINITY;
    float m = fmaxf(l0, l1);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((t & 63) == 0) red[0][wv] = m;
    __syncthreads();
    const float M = fmaxf(red[0][0], red[0][1]);
    const float a0 = (M == -INFINITY || l0 == -INFINITY) ? 0.f : fast_exp2(l0 - M);
    const float a1 = (M == -INFINITY || l1 == -INFINITY) ? 0.f : fast_exp2(l1 - M);
    wgt[t] = a0;
    wgt[t + kD] = a1;
    float sum = a0 + a1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if ((t & 63) == 0) red[1][wv] = sum;
    __syncthreads();
    const float L = red[1][0] + red[1][1];
    const float* col = ws + r * kD + t;
    const int64_t stride = R * kD;
    float acc = 0.f;
#pragma unroll 8
    for (int sp = 0; sp < n_splits; ++sp) acc += wgt[sp] * col[sp * stride];
    const float o = L > 0.f ? acc / L : 0.f;
    reinterpret_cast<__bf16*>(p.o)[r * kD + t] = static_cast<__bf16>(o);
    if (t == 0 && p.lse != nullptr) p.lse[r] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

bool decode_applies(const FwdParams& p, int d, bool is_bf16) {
    return is_bf16 && d == kD && p.Nq <= 16;
}

hipError_t launch_fwd_decode(const FwdParams& p, bool causal, hipStream_t stream) {
    return launch_fwd_decode_split(p, causal, 1, nullptr, stream);
}

hipError_t launch_fwd_decode_split(const FwdParams& p, bool causal, int n_splits, float* ws, hipStream_t stream) {
    const long long row_tiles = ((long long)p.Nq * p.group + 31) / 32;
    const long long grid = row_tiles * p.B * p.Hkv * n_splits;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    FwdParams pp = p;
    int c = causal ? 1 : 0;
    int ns = n_splits;
    float* w = ws;
    void* args[] = {&pp, &c, &ns, &w};
    const void* kernel = reinterpret_cast<const void*>(&fa_fwd_decode_kernel);
    hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(256), args, test_extra_lds(kLDS), stream);
    if (e != hipSuccess || n_splits == 1) return e;
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    if (rows > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    void* margs[] = {&pp, &ns, &w};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fa_decode_merge_kernel), dim3((unsigned)rows), dim3(kD),
                           margs, 0, stream);
}

}  // namespace fa
