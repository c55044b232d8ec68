// Gated DeltaNet scan with the state in registers, gfx950.
//
// Thirty of the model's 40 layers run Gated DeltaNet, a fixed-size recurrent state
// per head ("Perplexity built an inference engine for one model, one chip",
// paragraph 2); keeping that state in registers through the scan sped up prefill
// ("Perplexity's Lily brings fast local AI to Apple silicon Macs", section "Where
// the Engine Gains Speed").  Per value head h (query/key head c = h / rep), state S
// (128 value rows x 128 key columns, fp32), for each token:
//     a = exp(g_t);  S <- a S + beta_t (v_t - a S k_t) k_t^T;  o_t = S q_t
// which, per value row i, needs only that row:
//     dk = S_i . k,  dq = S_i . q,  c = beta (v_i - a dk)
//     o_i = a dq + c (k . q),  S_i <- a S_i + c k
// (the read S_t q uses the updated row; expanding it gives a dq + c k.q).
//
// k_gdn_scan: grid (value heads, 8), four wavefronts.  A workgroup owns 16 value
// rows of one head; 16 lanes share a row, 8 key columns each, so a row's state is
// 8 registers per lane for the whole sequence and the two dots are DPP row sums.
// Tokens are processed in chunks of 32: q and k (fp32), k . q, a, beta and the
// workgroup's v entries are staged in LDS first, the 32 sequential steps run from
// LDS, and the chunk's outputs leave as one coalesced bf16 store.
#include "device.h"
#include "kernels.h"

namespace moe_w4 {

constexpr int kGdnD = 128;
constexpr int kGdnRows = 16;        // value rows per workgroup
constexpr int kGdnTC = 32;          // tokens per staged chunk

__global__ __launch_bounds__(256) void k_gdn_scan(GdnArgs a) {
    __shared__ float s_k[kGdnTC][kGdnD];
    __shared__ float s_q[kGdnTC][kGdnD];
    __shared__ float s_v[kGdnTC][kGdnRows];
    __shared__ float s_o[kGdnTC][kGdnRows];
    __shared__ float s_a[kGdnTC], s_b[kGdnTC], s_kq[kGdnTC];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int h = blockIdx.x;
    const int c = h / a.rep;
    const int r0 = blockIdx.y * kGdnRows;
    const int rl = wave * 4 + (lane >> 4);          // this lane's row within the workgroup
    const int col = (lane & 15) * 8;                // its 8 key columns
    float* srow = a.state + ((size_t)h * kGdnD + r0 + rl) * kGdnD + col;
    float S[8];
    {
        const float4 x0 = *reinterpret_cast<const float4*>(srow);
        const float4 x1 = *reinterpret_cast<const float4*>(srow + 4);
        S[0] = x0.x; S[1] = x0.y; S[2] = x0.z; S[3] = x0.w;
        S[4] = x1.x; S[5] = x1.y; S[6] = x1.z; S[7] = x1.w;
    }
    const int T = a.T;
    for (int t0 = 0; t0 < T; t0 += kGdnTC) {
        const int nt = min(kGdnTC, T - t0);
        // stage: q, k (bf16 -> fp32), 8 columns per thread per item
        for (int i = threadIdx.x; i < nt * (kGdnD / 8); i += blockDim.x) {
            const int t = i / (kGdnD / 8), j = (i - t * (kGdnD / 8)) * 8;
            const size_t off = ((size_t)(t0 + t) * a.Hk + c) * kGdnD + j;
            const u32x4 kk = load_u32x4(a.k + off);
            const u32x4 qq = load_u32x4(a.q + off);
            const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w}, qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s_k[t][j + 2 * e] = __uint_as_float(kw[e] << 16);
                s_k[t][j + 2 * e + 1] = __uint_as_float(kw[e] & 0xFFFF0000u);
                s_q[t][j + 2 * e] = __uint_as_float(qw[e] << 16);
                s_q[t][j + 2 * e + 1] = __uint_as_float(qw[e] & 0xFFFF0000u);
            }
        }
        for (int i = threadIdx.x; i < nt * kGdnRows; i += blockDim.x) {
            const int t = i / kGdnRows, r = i - t * kGdnRows;
            const uint16_t vb = a.v[((size_t)(t0 + t) * a.Hv + h) * kGdnD + r0 + r];
            s_v[t][r] = __uint_as_float((uint32_t)vb << 16);
        }
        for (int t = threadIdx.x; t < nt; t += blockDim.x) {
            const size_t gi = (size_t)(t0 + t) * a.Hv + h;
            s_a[t] = __expf(a.g[gi]);
            s_b[t] = a.beta[gi];
        }
        __syncthreads();
        // k . q per token: wavefront w takes tokens w, w + 4, ...
        for (int t = wave; t < nt; t += 4) {
            float p = s_k[t][lane] * s_q[t][lane] + s_k[t][lane + 64] * s_q[t][lane + 64];
            p = wave_sum(p);
            if (lane == 0) s_kq[t] = p;
        }
        __syncthreads();
        // the sequential steps: the next token's operands are read from LDS while
        // the current token's dependent chain (dots, row sums, update) runs
        struct Tok {
            float k[8], q[8];
            float al, b, v, kq;
        };
        auto fetch = [&](Tok& o, int t) {
            const float4 k0 = *reinterpret_cast<const float4*>(&s_k[t][col]);
            const float4 k1 = *reinterpret_cast<const float4*>(&s_k[t][col + 4]);
            const float4 q0 = *reinterpret_cast<const float4*>(&s_q[t][col]);
            const float4 q1 = *reinterpret_cast<const float4*>(&s_q[t][col + 4]);
            o.k[0] = k0.x; o.k[1] = k0.y; o.k[2] = k0.z; o.k[3] = k0.w;
            o.k[4] = k1.x; o.k[5] = k1.y; o.k[6] = k1.z; o.k[7] = k1.w;
            o.q[0] = q0.x; o.q[1] = q0.y; o.q[2] = q0.z; o.q[3] = q0.w;
            o.q[4] = q1.x; o.q[5] = q1.y; o.q[6] = q1.z; o.q[7] = q1.w;
            o.al = s_a[t];
            o.b = s_b[t];
            o.v = s_v[t][rl];
            o.kq = s_kq[t];
        };
        auto step = [&](const Tok& x, int t) {
            float dk0 = 0.f, dk1 = 0.f, dq0 = 0.f, dq1 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                dk0 = fmaf(S[e], x.k[e], dk0);
                dk1 = fmaf(S[e + 1], x.k[e + 1], dk1);
                dq0 = fmaf(S[e], x.q[e], dq0);
                dq1 = fmaf(S[e + 1], x.q[e + 1], dq1);
            }
            const float dk = row16_sum(dk0 + dk1);
            const float dq = row16_sum(dq0 + dq1);
            const float cc = x.b * (x.v - x.al * dk);
#pragma unroll
            for (int e = 0; e < 8; ++e) S[e] = fmaf(x.al, S[e], cc * x.k[e]);
            if ((lane & 15) == 0) s_o[t][rl] = fmaf(x.al, dq, cc * x.kq);
        };
        // two tokens per iteration, alternating operand sets (no register copies)
        Tok ta, tb;
        fetch(ta, 0);
        int t = 0;
        for (; t + 1 < nt; t += 2) {
            fetch(tb, t + 1);
            step(ta, t);
            fetch(ta, min(t + 2, nt - 1));
            step(tb, t + 1);
        }
        if (t < nt) step(ta, t);
        __syncthreads();
        // outputs: bf16 pairs, 32 bytes per token
        for (int i = threadIdx.x; i < nt * (kGdnRows / 2); i += blockDim.x) {
            const int t = i / (kGdnRows / 2), r = (i - t * (kGdnRows / 2)) * 2;
            uint32_t* dst = reinterpret_cast<uint32_t*>(a.out + ((size_t)(t0 + t) * a.Hv + h) * kGdnD + r0 + r);
            *dst = pack_bf16x2(s_o[t][r], s_o[t][r + 1]);
        }
        __syncthreads();      // the next chunk overwrites the staging arrays
    }
    *reinterpret_cast<float4*>(srow) = float4{S[0], S[1], S[2], S[3]};
    *reinterpret_cast<float4*>(srow + 4) = float4{S[4], S[5], S[6], S[7]};
}

hipError_t launch_gdn_scan(const GdnArgs& a, hipStream_t st, KernelTimer& tm) {
    tm.before();
    tm.launch(k_gdn_scan, dim3(a.Hv, kGdnD / kGdnRows), dim3(256), 0, st, a);
    tm.after();
    return hipGetLastError();
}

}  // namespace moe_w4
