// Host side of the C ABI declared in include/w4a4.h: argument checks, then
// kernel launches on the caller's stream. Nothing here allocates device
// memory; all buffers belong to the caller.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "w4a4.h"
#include "quant_internal.h"
#include "w4a4_internal.h"
#include "w4a8_internal.h"
#include "gemm_fp6_internal.h"

namespace {

constexpr int64_t kAccLimit = int64_t(1) << 31;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape rules shared by every device call.
w4a4_status check_shape(int32_t rows, int32_t K, int32_t n_out, int32_t group) {
    if (rows < 0 || K <= 0 || n_out < 0 || n_out > K || group < 0)
        return W4A4_ERR_INVALID_ARG;
    const int32_t K_n = K - n_out;
    if (group > 0 && K_n % group != 0)
        return W4A4_ERR_INVALID_ARG;
    if (group % 128 != 0)                       // GPU kernels: 0 or multiples of 128
        return W4A4_ERR_UNSUPPORTED;
    // widened INT4 operands carry 16 x 16; |code product| <= 64 (INT4), 16384 (INT8)
    if ((int64_t)K_n * 64 * 256 >= kAccLimit || (int64_t)n_out * 16384 >= kAccLimit)
        return W4A4_ERR_UNSUPPORTED;
    return W4A4_OK;
}

// The GEMM kernels address operand rows by a 32-bit byte offset from the
// operand's base (row * pitch + column), so every packed row must start below
// 4 GiB.
bool dma_offsets_fit(int64_t M, int64_t N, int32_t K_n, int32_t n_out) {
    const int64_t rows = M > N ? M : N;
    const int64_t pitch = std::max(w4a4_pitch4_bytes(K_n), w4a4_pitch8_bytes(n_out));
    return rows * pitch < (int64_t(1) << 32);
}

// Optional RMSNorm in front of the quantizer (gamma == nullptr: none).
struct NormArgs {
    const void *gamma;
    float eps;
    float *rstd;
};

// q4: packed nibbles [rows, pitch4]; or, with u6 set (q4 unused), the head
// as the FP6 GEMM's u6 operand (no norm).
w4a4_status quant_rows(const void *src, int64_t ld, const int32_t *perm, int32_t rows,
                       int32_t K, int32_t n_out, int32_t group, void *q4, void *q8, float *s4,
                       float *s8, w4a4_stream stream, const NormArgs &norm = NormArgs{nullptr, 0.0f, nullptr},
                       void *u6 = nullptr) {
    w4a4_status st = check_shape(rows, K, n_out, group);
    if (st != W4A4_OK)
        return st;
    const int32_t K_n = K - n_out;
    const int32_t G = w4a4_num_groups(K_n, group);
    if (ld < K)
        return W4A4_ERR_INVALID_ARG;
    if (rows == 0)
        return W4A4_OK;                         // empty call: pointers are not used
    if (!src)                                   // perm may be null: the identity order
        return W4A4_ERR_INVALID_ARG;
    if ((K_n > 0 && (!(u6 ? u6 : q4) || !s4)) || (n_out > 0 && (!q8 || !s8)))
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(src, 16) || ld % 8 != 0 || (perm && !aligned(perm, 16)) || (q4 && !aligned(q4, 16)) ||
        (u6 && !aligned(u6, 16)) || (q8 && !aligned(q8, 16)) || (s4 && !aligned(s4, 4)) || (s8 && !aligned(s8, 4)))
        return W4A4_ERR_ALIGNMENT;
    if (norm.gamma && (!aligned(norm.gamma, 2) || (norm.rstd && !aligned(norm.rstd, 4))))
        return W4A4_ERR_ALIGNMENT;
    w4a4::QuantArgs a;
    a.src = static_cast<const _Float16 *>(src);
    a.ld = ld;
    a.perm = perm;
    a.rows = rows;
    a.K = K;
    a.n_out = n_out;
    a.K_n = K_n;
    a.group = group;
    a.G = G;
    a.q4 = u6 ? nullptr : static_cast<uint8_t *>(q4);
    a.u6 = static_cast<uint8_t *>(u6);
    a.q8 = static_cast<int8_t *>(q8);
    a.s4 = s4;
    a.s8 = s8;
    a.pitch4 = w4a4_pitch4_bytes(K_n);
    a.pitch8 = n_out > 0 ? w4a4_pitch8_bytes(n_out) : 0;
    a.gamma = static_cast<const _Float16 *>(norm.gamma);
    a.eps = norm.eps;
    a.rstd = norm.gamma ? norm.rstd : nullptr;
    // the permutation and two row buffers live in LDS
    if (K > w4a4::quant_rows_max_k())
        return W4A4_ERR_UNSUPPORTED;
    if (w4a4::launch_quant_rows(a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

// Arguments of the norm that are checked before anything else.
w4a4_status norm_check(int32_t rows, const void *gamma, float eps) {
    if (!(eps >= 0.0f) || eps > 3.4028235e38f)    // negative, NaN or infinite
        return W4A4_ERR_INVALID_ARG;
    if (rows > 0 && !gamma)
        return W4A4_ERR_INVALID_ARG;
    return W4A4_OK;
}

w4a4_status gemm_check(const void *Aq4, const void *Aq8, const void *Wq4, const void *Wq8,
                       int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group) {
    if (N < 0)
        return W4A4_ERR_INVALID_ARG;
    w4a4_status st = check_shape(M, K, n_out, group);
    if (st != W4A4_OK)
        return st;
    const int32_t K_n = K - n_out;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if ((K_n > 0 && (!Aq4 || !Wq4)) || (n_out > 0 && (!Aq8 || !Wq8)))
        return W4A4_ERR_INVALID_ARG;
    if ((Aq4 && !aligned(Aq4, 16)) || (Wq4 && !aligned(Wq4, 16)) || (Aq8 && !aligned(Aq8, 16)) ||
        (Wq8 && !aligned(Wq8, 16)))
        return W4A4_ERR_ALIGNMENT;
    if (!dma_offsets_fit(M, N, K_n, n_out))
        return W4A4_ERR_UNSUPPORTED;
    return W4A4_OK;
}

w4a4::GemmArgs gemm_args(const void *Aq4, const void *Aq8, const float *sa4, const float *sa8,
                         const void *Wq4, const void *Wq8, const float *sw4, const float *sw8,
                         int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group) {
    w4a4::GemmArgs a;
    memset(&a, 0, sizeof(a));
    const int32_t K_n = K - n_out;
    a.a4 = static_cast<const uint8_t *>(Aq4);
    a.a8 = static_cast<const int8_t *>(Aq8);
    a.w4 = static_cast<const uint8_t *>(Wq4);
    a.w8 = static_cast<const int8_t *>(Wq8);
    a.sa4 = sa4;
    a.sa8 = sa8;
    a.sw4 = sw4;
    a.sw8 = sw8;
    a.M = M;
    a.N = N;
    a.K_n = K_n;
    a.n_out = n_out;
    a.group = group;
    a.G = w4a4_num_groups(K_n, group);
    a.pitch4 = w4a4_pitch4_bytes(K_n);
    a.pitch8 = n_out > 0 ? w4a4_pitch8_bytes(n_out) : 0;
    return a;
}

}  // namespace

extern "C" {

const char *w4a4_status_string(int status) {
    switch (status) {
    case W4A4_OK: return "W4A4_OK";
    case W4A4_ERR_INVALID_ARG: return "W4A4_ERR_INVALID_ARG";
    case W4A4_ERR_UNSUPPORTED: return "W4A4_ERR_UNSUPPORTED";
    case W4A4_ERR_ALIGNMENT: return "W4A4_ERR_ALIGNMENT";
    case W4A4_ERR_HIP: return "W4A4_ERR_HIP";
    case W4A4_ERR_WORKSPACE: return "W4A4_ERR_WORKSPACE";
    default: return "W4A4_ERR_UNKNOWN";
    }
}

int32_t w4a4_num_groups(int32_t K_n, int32_t group) {
    if (K_n < 0 || group < 0 || (group > 0 && K_n % group != 0))
        return -1;
    if (K_n == 0)
        return 0;
    return group > 0 ? K_n / group : 1;
}

int64_t w4a4_pitch4_bytes(int32_t K_n) { return K_n <= 0 ? 0 : round_up(K_n, 128) / 2; }

int64_t w4a4_pitch8_bytes(int32_t n_out) { return n_out <= 0 ? 0 : round_up(n_out, 64); }

w4a4_status w4a4_make_perm(int32_t K, const int32_t *outlier_idx, int32_t n_out, int32_t *perm) {
    if (K <= 0 || n_out < 0 || n_out > K || !perm || (n_out > 0 && !outlier_idx))
        return W4A4_ERR_INVALID_ARG;
    std::vector<unsigned char> is_out(K, 0);
    for (int32_t i = 0; i < n_out; ++i) {
        const int32_t c = outlier_idx[i];
        if (c < 0 || c >= K || is_out[c])
            return W4A4_ERR_INVALID_ARG;
        is_out[c] = 1;
    }
    int32_t head = 0, tail = K - n_out;
    for (int32_t j = 0; j < K; ++j)
        perm[is_out[j] ? tail++ : head++] = j;
    return W4A4_OK;
}

w4a4_status w4a4_quant_reorder_act(const void *X, int64_t ldx, const int32_t *perm, int32_t M,
                                   int32_t K, int32_t n_out, int32_t group, void *Aq4, void *Aq8,
                                   float *sa4, float *sa8, w4a4_stream stream) {
    return quant_rows(X, ldx, perm, M, K, n_out, group, Aq4, Aq8, sa4, sa8, stream);
}

w4a4_status w4a4_rmsnorm_quant_reorder_act(const void *X, int64_t ldx, const void *gamma, float eps,
                                           const int32_t *perm, int32_t M, int32_t K, int32_t n_out,
                                           int32_t group, void *Aq4, void *Aq8, float *sa4, float *sa8,
                                           float *rstd, w4a4_stream stream) {
    w4a4_status st = norm_check(M, gamma, eps);
    if (st != W4A4_OK)
        return st;
    return quant_rows(X, ldx, perm, M, K, n_out, group, Aq4, Aq8, sa4, sa8, stream,
                      NormArgs{gamma, eps, rstd});
}

w4a4_status w4a4_pack_int4_weights(const void *W, int64_t ldw, const int32_t *perm, int32_t N,
                                   int32_t K, int32_t n_out, int32_t group, void *Wq4, void *Wq8,
                                   float *sw4, float *sw8, w4a4_stream stream) {
    return quant_rows(W, ldw, perm, N, K, n_out, group, Wq4, Wq8, sw4, sw8, stream);
}

size_t w4a4_outlier_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                         int32_t group) {
    if (M <= 0 || N <= 0 || K <= 0 || n_out < 0 || n_out > K || w4a4_num_groups(K - n_out, group) < 0)
        return 0;
    return w4a4::plan_gemm(M, N, K - n_out, n_out, group).workspace_bytes;
}

const char *w4a4_outlier_gemm_kernel_name(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group) {
    if (M <= 0 || N <= 0 || K <= 0 || n_out < 0 || n_out > K || w4a4_num_groups(K - n_out, group) < 0)
        return nullptr;
    return w4a4::gemm_kernel_name(w4a4::plan_gemm(M, N, K - n_out, n_out, group));
}

const char *w4a4_quant_gemm_kernel_name(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group) {
    if (M > 0 && N > 0 && w4a4::decode_fused_fits(M, N, K, n_out, group))
        return "decode_fused_kernel";
    return w4a4_outlier_gemm_kernel_name(M, N, K, n_out, group);
}

}  // extern "C"

static w4a4_status outlier_gemm(const void *Aq4, const void *Aq8, const float *sa4, const float *sa8,
                                const void *Wq4, const void *Wq8, const float *sw4, const float *sw8,
                                int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                                int64_t ldy, void *workspace, size_t workspace_bytes, int32_t *acc4,
                                int32_t *acc8, bool export_acc, w4a4_stream stream) {
    w4a4_status st = gemm_check(Aq4, Aq8, Wq4, Wq8, M, N, K, n_out, group);
    if (st != W4A4_OK)
        return st;
    const int32_t K_n = K - n_out;
    if (ldy < N)
        return W4A4_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if (!Y || (K_n > 0 && (!sa4 || !sw4)) || (n_out > 0 && (!sa8 || !sw8)))
        return W4A4_ERR_INVALID_ARG;
    if (export_acc && ((K_n > 0 && !acc4) || (n_out > 0 && !acc8)))
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(Y, 2) || (sa4 && !aligned(sa4, 4)) || (sw4 && !aligned(sw4, 4)) ||
        (sa8 && !aligned(sa8, 4)) || (sw8 && !aligned(sw8, 4)) ||
        (export_acc && ((acc4 && !aligned(acc4, 4)) || (acc8 && !aligned(acc8, 4)))))
        return W4A4_ERR_ALIGNMENT;
    const size_t need = w4a4_outlier_gemm_workspace_bytes(M, N, K, n_out, group);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return W4A4_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 256))
        return W4A4_ERR_ALIGNMENT;
    w4a4::GemmArgs a = gemm_args(Aq4, Aq8, sa4, sa8, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group);
    a.y = static_cast<_Float16 *>(Y);
    a.ldy = ldy;
    if (export_acc) {
        a.acc4_out = K_n > 0 ? acc4 : nullptr;
        a.acc8_out = n_out > 0 ? acc8 : nullptr;
    }
    if (w4a4::launch_gemm(a, export_acc, workspace, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

extern "C" {

w4a4_status w4a4_outlier_gemm(const void *Aq4, const void *Aq8, const float *sa4, const float *sa8,
                              const void *Wq4, const void *Wq8, const float *sw4, const float *sw8,
                              int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group,
                              void *Y, int64_t ldy, void *workspace, size_t workspace_bytes,
                              w4a4_stream stream) {
    return outlier_gemm(Aq4, Aq8, sa4, sa8, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, workspace,
                        workspace_bytes, nullptr, nullptr, false, stream);
}

w4a4_status w4a4_outlier_gemm_i32(const void *Aq4, const void *Aq8, const float *sa4, const float *sa8,
                                  const void *Wq4, const void *Wq8, const float *sw4, const float *sw8,
                                  int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group,
                                  void *Y, int64_t ldy, void *workspace, size_t workspace_bytes,
                                  int32_t *acc4, int32_t *acc8, w4a4_stream stream) {
    return outlier_gemm(Aq4, Aq8, sa4, sa8, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, workspace,
                        workspace_bytes, acc4, acc8, true, stream);
}

// Workspace of the fused call: first the GEMM's own workspace, whose
// arrival-counter block always sits at offset 0 and is always reserved (also
// for shapes that do not split K), so the activation operands of one call
// never land on the counters of a later one; then Aq4 | Aq8 | sa4 | sa8,
// each 256-byte aligned. off[0..3] are the operand offsets, off[4] the size.
static void quant_gemm_layout(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group, size_t off[5]) {
    const int32_t K_n = K - n_out;
    const int32_t G = w4a4_num_groups(K_n, group);
    const size_t gemm = std::max(w4a4_outlier_gemm_workspace_bytes(M, N, K, n_out, group), w4a4::gemm_counter_bytes());
    off[0] = round_up((int64_t)gemm, 256);
    off[1] = off[0] + round_up((int64_t)M * w4a4_pitch4_bytes(K_n), 256);
    off[2] = off[1] + round_up((int64_t)M * w4a4_pitch8_bytes(n_out), 256);
    off[3] = off[2] + round_up((int64_t)M * (G > 0 ? G : 0) * 4, 256);
    off[4] = off[3] + round_up((int64_t)M * 4, 256);
}

size_t w4a4_quant_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                       int32_t group) {
    if (M < 0 || K <= 0 || n_out < 0 || n_out > K || w4a4_num_groups(K - n_out, group) < 0)
        return 0;
    size_t off[5];
    quant_gemm_layout(M, N, K, n_out, group, off);
    return off[4];
}

}  // extern "C"

static w4a4_status quant_gemm(const void *X, int64_t ldx, const int32_t *perm, const void *Wq4,
                              const void *Wq8, const float *sw4, const float *sw8, int32_t M,
                              int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                              int64_t ldy, void *workspace, size_t workspace_bytes,
                              w4a4_stream stream, const NormArgs &norm, bool clear_counters = false) {
    if (N < 0)
        return W4A4_ERR_INVALID_ARG;
    w4a4_status st = check_shape(M, K, n_out, group);
    if (st != W4A4_OK)
        return st;
    const int32_t K_n = K - n_out;
    if (ldx < K || ldy < N)
        return W4A4_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if (!dma_offsets_fit(M, N, K_n, n_out))
        return W4A4_ERR_UNSUPPORTED;
    if (!X || !perm || !Y || (K_n > 0 && (!Wq4 || !sw4)) ||
        (n_out > 0 && (!Wq8 || !sw8)))
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(X, 16) || ldx % 8 != 0 || !aligned(perm, 16) || !aligned(Y, 2) ||
        (Wq4 && !aligned(Wq4, 16)) || (Wq8 && !aligned(Wq8, 16)) || (sw4 && !aligned(sw4, 4)) ||
        (sw8 && !aligned(sw8, 4)) || !aligned(workspace, 256))
        return W4A4_ERR_ALIGNMENT;
    const size_t need = w4a4_quant_gemm_workspace_bytes(M, N, K, n_out, group);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return W4A4_ERR_WORKSPACE;
    if (K > w4a4::quant_rows_max_k())            // the producer's longest row (checked before any launch)
        return W4A4_ERR_UNSUPPORTED;
    // small decode batches: the quantizer (and the norm, for one token: a
    // second row already costs more than the norm producer's launch) run
    // inside the GEMM's workgroups
    if (w4a4::decode_fused_fits(M, N, K, n_out, group) && (!norm.gamma || M == 1)) {
        w4a4::DecodeFusedArgs f{};
        f.x = static_cast<const uint16_t *>(X);
        f.gamma = static_cast<const uint16_t *>(norm.gamma);
        f.eps = norm.eps;
        f.perm = perm;
        f.w4 = static_cast<const uint8_t *>(Wq4);
        f.w8 = static_cast<const int8_t *>(Wq8);
        f.sw4 = sw4;
        f.sw8 = sw8;
        f.y = static_cast<_Float16 *>(Y);
        f.M = M;
        f.N = N;
        f.K = K;
        f.K_n = K_n;
        f.n_out = n_out;
        f.ldx = ldx;
        f.pitch4 = w4a4_pitch4_bytes(K_n);
        f.pitch8 = w4a4_pitch8_bytes(n_out);
        f.ldy = ldy;
        return w4a4::launch_decode_fused(f, static_cast<hipStream_t>(stream)) == hipSuccess ? W4A4_OK
                                                                                        : W4A4_ERR_HIP;
    }
    size_t off[5];
    quant_gemm_layout(M, N, K, n_out, group, off);
    char *ws = static_cast<char *>(workspace);
    // a workspace that keeps earlier contents (the static one) gets its
    // split-K arrival counters cleared first, by a kernel on the stream
    if (clear_counters && w4a4_outlier_gemm_workspace_bytes(M, N, K, n_out, group) > 0 &&
        w4a4::clear_gemm_counters(ws, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    void *Aq4 = K_n > 0 ? ws + off[0] : nullptr;
    void *Aq8 = n_out > 0 ? ws + off[1] : nullptr;
    float *sa4 = K_n > 0 ? reinterpret_cast<float *>(ws + off[2]) : nullptr;
    float *sa8 = reinterpret_cast<float *>(ws + off[3]);
    st = quant_rows(X, ldx, perm, M, K, n_out, group, Aq4, Aq8, sa4, sa8, stream, norm);
    if (st != W4A4_OK)
        return st;
    return w4a4_outlier_gemm(Aq4, Aq8, sa4, sa8, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy,
                             ws, off[0], stream);
}

extern "C" {

w4a4_status w4a4_quant_gemm(const void *X, int64_t ldx, const int32_t *perm, const void *Wq4,
                            const void *Wq8, const float *sw4, const float *sw8, int32_t M,
                            int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                            int64_t ldy, void *workspace, size_t workspace_bytes,
                            w4a4_stream stream) {
    return quant_gemm(X, ldx, perm, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, workspace,
                      workspace_bytes, stream, NormArgs{nullptr, 0.0f, nullptr});
}

static w4a4_status w4a8_check(const void *Aq8, const void *Wq4, int32_t M, int32_t N, int32_t K,
                              int32_t group) {
    if (M < 0 || N < 0 || K <= 0 || group < 0 || (group > 0 && K % group != 0))
        return W4A4_ERR_INVALID_ARG;
    if (K % 128 != 0 || group % 128 != 0 || (int64_t)K * 16384 >= kAccLimit)
        return W4A4_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if (!Aq8 || !Wq4)
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(Aq8, 16) || !aligned(Wq4, 16))
        return W4A4_ERR_ALIGNMENT;
    return W4A4_OK;
}

static w4a4::GemmArgs w4a8_args(const void *Aq8, const float *sa8, const void *Wq4, const float *sw4,
                                int32_t M, int32_t N, int32_t K, int32_t group) {
    w4a4::GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.a8 = static_cast<const int8_t *>(Aq8);
    a.w4 = static_cast<const uint8_t *>(Wq4);
    a.sa8 = sa8;
    a.sw4 = sw4;
    a.M = M;
    a.N = N;
    a.K_n = K;
    a.group = group;
    a.G = w4a4_num_groups(K, group);
    a.pitch4 = w4a4_pitch4_bytes(K);
    a.pitch8 = w4a4_pitch8_bytes(K);
    return a;
}

w4a4_status w4a4_w4a8_gemm(const void *Aq8, const float *sa8, const void *Wq4, const float *sw4,
                           int32_t M, int32_t N, int32_t K, int32_t group, void *Y, int64_t ldy,
                           w4a4_stream stream) {
    w4a4_status st = w4a8_check(Aq8, Wq4, M, N, K, group);
    if (st != W4A4_OK)
        return st;
    if (ldy < N)
        return W4A4_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if (!sa8 || !sw4 || !Y)
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(sa8, 4) || !aligned(sw4, 4) || !aligned(Y, 2))
        return W4A4_ERR_ALIGNMENT;
    w4a4::GemmArgs a = w4a8_args(Aq8, sa8, Wq4, sw4, M, N, K, group);
    a.y = static_cast<_Float16 *>(Y);
    a.ldy = ldy;
    if (w4a4::launch_gemm_w4a8(a, false, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

w4a4_status w4a4_w4a8_gemm_i32(const void *Aq8, const void *Wq4, int32_t M, int32_t N, int32_t K,
                               int32_t group, int32_t *acc, w4a4_stream stream) {
    w4a4_status st = w4a8_check(Aq8, Wq4, M, N, K, group);
    if (st != W4A4_OK)
        return st;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if (!acc)
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(acc, 4))
        return W4A4_ERR_ALIGNMENT;
    w4a4::GemmArgs a = w4a8_args(Aq8, nullptr, Wq4, nullptr, M, N, K, group);
    a.acc4_out = acc;
    if (w4a4::launch_gemm_w4a8(a, true, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

static w4a4_status kv_check(int32_t T, int32_t H, int32_t D, int32_t bits, int64_t num_slots,
                            const void *cache_q, const float *cache_s, const int32_t *slots) {
    if (T < 0 || H < 0 || num_slots < 0 || (bits != 4 && bits != 8))
        return W4A4_ERR_INVALID_ARG;
    if (D != 64 && D != 128 && D != 256)
        return W4A4_ERR_UNSUPPORTED;
    if ((int64_t)T * H == 0)
        return W4A4_OK;
    if (num_slots < 1 || !cache_q || !cache_s || (!slots && num_slots < T))
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(cache_q, 16) || !aligned(cache_s, 4) || (slots && !aligned(slots, 4)))
        return W4A4_ERR_ALIGNMENT;
    return W4A4_OK;
}

w4a4_status w4a4_kv_quant(const void *X, int64_t ldx, int32_t T, int32_t H, int32_t D, int32_t bits,
                          const int32_t *slot_mapping, int64_t num_slots, void *cache_q, float *cache_s,
                          w4a4_stream stream) {
    w4a4_status st = kv_check(T, H, D, bits, num_slots, cache_q, cache_s, slot_mapping);
    if (st != W4A4_OK)
        return st;
    if (ldx < (int64_t)H * D)
        return W4A4_ERR_INVALID_ARG;
    if ((int64_t)T * H == 0)
        return W4A4_OK;
    if (!X)
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(X, 16) || ldx % 8 != 0)
        return W4A4_ERR_ALIGNMENT;
    w4a4::KvArgs a;
    memset(&a, 0, sizeof(a));
    a.X = static_cast<const _Float16 *>(X);
    a.ldx = ldx;
    a.T = T;
    a.H = H;
    a.D = D;
    a.bits = bits;
    a.slots = slot_mapping;
    a.num_slots = num_slots;
    a.cq = static_cast<uint8_t *>(cache_q);
    a.cs = cache_s;
    if (w4a4::launch_kv(a, true, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

w4a4_status w4a4_kv_dequant(const void *cache_q, const float *cache_s, int64_t num_slots,
                            const int32_t *slot_mapping, int32_t T, int32_t H, int32_t D, int32_t bits,
                            void *Y, int64_t ldy, w4a4_stream stream) {
    w4a4_status st = kv_check(T, H, D, bits, num_slots, cache_q, cache_s, slot_mapping);
    if (st != W4A4_OK)
        return st;
    if (ldy < (int64_t)H * D)
        return W4A4_ERR_INVALID_ARG;
    if ((int64_t)T * H == 0)
        return W4A4_OK;
    if (!Y)
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(Y, 16) || ldy % 8 != 0)
        return W4A4_ERR_ALIGNMENT;
    w4a4::KvArgs a;
    memset(&a, 0, sizeof(a));
    a.Y = static_cast<_Float16 *>(Y);
    a.ldy = ldy;
    a.T = T;
    a.H = H;
    a.D = D;
    a.bits = bits;
    a.slots = slot_mapping;
    a.num_slots = num_slots;
    a.cq = static_cast<uint8_t *>(const_cast<void *>(cache_q));
    a.cs = const_cast<float *>(cache_s);
    if (w4a4::launch_kv(a, false, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

size_t w4a4_select_outliers_workspace_bytes(int32_t rows, int32_t K) {
    if (rows < 0 || K <= 0 || K > w4a4::select_max_k())
        return 0;
    return w4a4::plan_select(rows, K).workspace_bytes;
}

w4a4_status w4a4_select_outliers(const void *Xcal, int64_t ldx, int32_t rows, int32_t K,
                                 int32_t n_out, int32_t *outlier_idx, int32_t *perm,
                                 void *chan_absmax, void *workspace, size_t workspace_bytes,
                                 w4a4_stream stream) {
    if (rows < 0 || K <= 0 || n_out < 0 || n_out > K || ldx < K)
        return W4A4_ERR_INVALID_ARG;
    if (K > w4a4::select_max_k())
        return W4A4_ERR_UNSUPPORTED;
    if (!perm || (n_out > 0 && !outlier_idx) || (rows > 0 && !Xcal))
        return W4A4_ERR_INVALID_ARG;
    if ((rows > 0 && (!aligned(Xcal, 16) || ldx % 8 != 0)) || !aligned(perm, 4) ||
        (outlier_idx && !aligned(outlier_idx, 4)) || (chan_absmax && !aligned(chan_absmax, 2)))
        return W4A4_ERR_ALIGNMENT;
    const size_t need = w4a4_select_outliers_workspace_bytes(rows, K);
    if (workspace_bytes < need || !workspace)
        return W4A4_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return W4A4_ERR_ALIGNMENT;
    w4a4::SelectArgs a;
    a.X = Xcal;
    a.ld = ldx;
    a.rows = rows;
    a.K = K;
    a.n_out = n_out;
    a.outlier_idx = n_out > 0 ? outlier_idx : nullptr;
    a.perm = perm;
    a.absmax = chan_absmax;
    a.workspace = workspace;
    if (w4a4::launch_select(a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

w4a4_status w4a4_rmsnorm_quant_gemm(const void *X, int64_t ldx, const void *gamma, float eps,
                                    const int32_t *perm, const void *Wq4, const void *Wq8,
                                    const float *sw4, const float *sw8, int32_t M, int32_t N,
                                    int32_t K, int32_t n_out, int32_t group, void *Y, int64_t ldy,
                                    void *workspace, size_t workspace_bytes, w4a4_stream stream) {
    w4a4_status st = norm_check(M, gamma, eps);
    if (st != W4A4_OK)
        return st;
    return quant_gemm(X, ldx, perm, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, workspace,
                      workspace_bytes, stream, NormArgs{gamma, eps, nullptr});
}

// ---------------------------------------------------------------------------
// FP6 prefill GEMM
// ---------------------------------------------------------------------------

int64_t w4a4_u6_bytes(int32_t rows, int32_t K_n) {
    if (rows < 0 || K_n < 0)
        return -1;
    return w4a4::u6_operand_bytes(rows, w4a4_pitch4_bytes(K_n));
}

w4a4_status w4a4_repack_u6(const void *Q4, int32_t rows, int32_t K_n, void *U6, w4a4_stream stream) {
    if (rows < 0 || K_n < 0)
        return W4A4_ERR_INVALID_ARG;
    const int64_t p4 = w4a4_pitch4_bytes(K_n);
    if ((int64_t)rows * p4 == 0)
        return W4A4_OK;
    if (!Q4 || !U6)
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(Q4, 16) || !aligned(U6, 16))
        return W4A4_ERR_ALIGNMENT;
    if (w4a4::launch_repack_u6(static_cast<const uint8_t *>(Q4), rows, p4, static_cast<uint8_t *>(U6),
                               static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

w4a4_status w4a4_quant_reorder_act_u6(const void *X, int64_t ldx, const int32_t *perm, int32_t M, int32_t K,
                                      int32_t n_out, int32_t group, void *Au6, void *Aq8, float *sa4,
                                      float *sa8, w4a4_stream stream) {
    return quant_rows(X, ldx, perm, M, K, n_out, group, nullptr, Aq8, sa4, sa8, stream,
                      NormArgs{nullptr, 0.0f, nullptr}, Au6);
}

w4a4_status w4a4_rmsnorm_quant_reorder_act_u6(const void *X, int64_t ldx, const void *gamma, float eps,
                                              const int32_t *perm, int32_t M, int32_t K, int32_t n_out,
                                              int32_t group, void *Au6, void *Aq8, float *sa4, float *sa8,
                                              float *rstd, w4a4_stream stream) {
    w4a4_status st = norm_check(M, gamma, eps);
    if (st != W4A4_OK)
        return st;
    return quant_rows(X, ldx, perm, M, K, n_out, group, nullptr, Aq8, sa4, sa8, stream,
                      NormArgs{gamma, eps, rstd}, Au6);
}

const char *w4a4_outlier_gemm_fp6_kernel_name(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group) {
    if (M <= 0 || N <= 0 || K <= 0 || n_out < 0 || n_out > K || w4a4_num_groups(K - n_out, group) < 0)
        return nullptr;
    return w4a4::gemm_fp6_kernel_name(M, N, K - n_out, n_out, group);
}

}  // extern "C"

static w4a4_status fp6_gemm(const void *Au6, const void *Aq8, const float *sa4, const float *sa8,
                            const void *Wu6, const void *Wq8, const float *sw4, const float *sw8, int32_t M,
                            int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y, int64_t ldy,
                            int32_t *acc4, int32_t *acc8, bool export_acc, w4a4_stream stream) {
    w4a4_status st = gemm_check(Au6, Aq8, Wu6, Wq8, M, N, K, n_out, group);
    if (st != W4A4_OK)
        return st;
    const int32_t K_n = K - n_out;
    if (ldy < N)
        return W4A4_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if (!w4a4::gemm_fp6_fits(M, N, K_n, n_out, group))
        return W4A4_ERR_UNSUPPORTED;
    if (!Y || !sa4 || !sw4 || (n_out > 0 && (!sa8 || !sw8)))
        return W4A4_ERR_INVALID_ARG;
    if (export_acc && (!acc4 || (n_out > 0 && !acc8)))
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(Y, 2) || !aligned(sa4, 4) || !aligned(sw4, 4) || (sa8 && !aligned(sa8, 4)) ||
        (sw8 && !aligned(sw8, 4)) || (export_acc && (!aligned(acc4, 4) || (acc8 && !aligned(acc8, 4)))))
        return W4A4_ERR_ALIGNMENT;
    const int64_t p4 = w4a4_pitch4_bytes(K_n);
    // u6 blocks are addressed by 32-bit offsets too
    if (w4a4_u6_bytes(M > N ? M : N, K_n) >= (int64_t(1) << 32))
        return W4A4_ERR_UNSUPPORTED;
    w4a4::Fp6GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.a_u6 = static_cast<const uint8_t *>(Au6);
    a.w_u6 = static_cast<const uint8_t *>(Wu6);
    a.a8 = static_cast<const int8_t *>(Aq8);
    a.w8 = static_cast<const int8_t *>(Wq8);
    a.sa4 = sa4;
    a.sa8 = sa8;
    a.sw4 = sw4;
    a.sw8 = sw8;
    a.y = static_cast<_Float16 *>(Y);
    a.acc4_out = export_acc ? acc4 : nullptr;
    a.acc8_out = export_acc && n_out > 0 ? acc8 : nullptr;
    a.M = M;
    a.N = N;
    a.K_n = K_n;
    a.n_out = n_out;
    a.pitch4 = p4;
    a.pitch8 = n_out > 0 ? w4a4_pitch8_bytes(n_out) : 0;
    a.ldy = ldy;
    if (w4a4::launch_gemm_fp6(a, group, export_acc, static_cast<hipStream_t>(stream)) != hipSuccess)
        return W4A4_ERR_HIP;
    return W4A4_OK;
}

extern "C" {

w4a4_status w4a4_outlier_gemm_fp6(const void *Au6, const void *Aq8, const float *sa4, const float *sa8,
                                  const void *Wu6, const void *Wq8, const float *sw4, const float *sw8,
                                  int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                                  int64_t ldy, w4a4_stream stream) {
    return fp6_gemm(Au6, Aq8, sa4, sa8, Wu6, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, nullptr, nullptr,
                    false, stream);
}

w4a4_status w4a4_outlier_gemm_fp6_i32(const void *Au6, const void *Aq8, const float *sa4, const float *sa8,
                                      const void *Wu6, const void *Wq8, const float *sw4, const float *sw8,
                                      int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                                      int64_t ldy, int32_t *acc4, int32_t *acc8, w4a4_stream stream) {
    return fp6_gemm(Au6, Aq8, sa4, sa8, Wu6, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, acc4, acc8, true,
                    stream);
}

// Workspace of the fused FP6 call: Au6 | Aq8 | sa4 | sa8, each 256-byte
// aligned; off[4] is the size.
static void quant_gemm_fp6_layout(int32_t M, int32_t K, int32_t n_out, int32_t group, size_t off[5]) {
    const int32_t K_n = K - n_out;
    const int32_t G = w4a4_num_groups(K_n, group);
    off[0] = 0;
    off[1] = off[0] + round_up(std::max<int64_t>(w4a4_u6_bytes(M, K_n), 0), 256);
    off[2] = off[1] + round_up((int64_t)M * w4a4_pitch8_bytes(n_out), 256);
    off[3] = off[2] + round_up((int64_t)M * (G > 0 ? G : 0) * 4, 256);
    off[4] = off[3] + round_up((int64_t)M * 4, 256);
}

size_t w4a4_quant_gemm_fp6_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n_out, int32_t group) {
    (void)N;
    if (M < 0 || K <= 0 || n_out < 0 || n_out > K || w4a4_num_groups(K - n_out, group) < 0)
        return 0;
    size_t off[5];
    quant_gemm_fp6_layout(M, K, n_out, group, off);
    return off[4];
}

w4a4_status w4a4_quant_gemm_fp6(const void *X, int64_t ldx, const int32_t *perm, const void *Wu6,
                                const void *Wq8, const float *sw4, const float *sw8, int32_t M, int32_t N,
                                int32_t K, int32_t n_out, int32_t group, void *Y, int64_t ldy, void *workspace,
                                size_t workspace_bytes, w4a4_stream stream) {
    if (N < 0)
        return W4A4_ERR_INVALID_ARG;
    w4a4_status st = check_shape(M, K, n_out, group);
    if (st != W4A4_OK)
        return st;
    const int32_t K_n = K - n_out;
    if (ldx < K || ldy < N)
        return W4A4_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return W4A4_OK;
    if (!w4a4::gemm_fp6_fits(M, N, K_n, n_out, group) || !dma_offsets_fit(M, N, K_n, n_out))
        return W4A4_ERR_UNSUPPORTED;
    if (!X || !perm || !Y || !Wu6 || !sw4 || (n_out > 0 && (!Wq8 || !sw8)))
        return W4A4_ERR_INVALID_ARG;
    if (!aligned(X, 16) || ldx % 8 != 0 || !aligned(perm, 16) || !aligned(Y, 2) || !aligned(Wu6, 16) ||
        (Wq8 && !aligned(Wq8, 16)) || !aligned(sw4, 4) || (sw8 && !aligned(sw8, 4)) || !aligned(workspace, 256))
        return W4A4_ERR_ALIGNMENT;
    const size_t need = w4a4_quant_gemm_fp6_workspace_bytes(M, N, K, n_out, group);
    if (workspace_bytes < need || !workspace)
        return W4A4_ERR_WORKSPACE;
    size_t off[5];
    quant_gemm_fp6_layout(M, K, n_out, group, off);
    char *ws = static_cast<char *>(workspace);
    void *Au6 = ws + off[0];
    void *Aq8 = n_out > 0 ? ws + off[1] : nullptr;
    float *sa4 = reinterpret_cast<float *>(ws + off[2]);
    float *sa8 = reinterpret_cast<float *>(ws + off[3]);
    st = quant_rows(X, ldx, perm, M, K, n_out, group, nullptr, Aq8, sa4, sa8, stream,
                    NormArgs{nullptr, 0.0f, nullptr}, Au6);
    if (st != W4A4_OK)
        return st;
    return w4a4_outlier_gemm_fp6(Au6, Aq8, sa4, sa8, Wu6, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The fused layer call without a caller workspace: for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its workspace is a file-scope device
// array, one copy per GPU, held until the process ends.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current (the host-side name is not a device address).
w4a4_status scratch_for_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return W4A4_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return W4A4_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return W4A4_OK;
}

}  // namespace

extern "C" {

size_t w4a4_quant_gemm_static_max_bytes(void) { return kScratchBytes; }

w4a4_status w4a4_quant_gemm_static(const void *X, int64_t ldx, const int32_t *perm, const void *Wq4,
                                   const void *Wq8, const float *sw4, const float *sw8, int32_t M, int32_t N,
                                   int32_t K, int32_t n_out, int32_t group, void *Y, int64_t ldy,
                                   w4a4_stream stream) {
    if (N < 0)
        return W4A4_ERR_INVALID_ARG;
    w4a4_status st = check_shape(M, K, n_out, group);
    if (st != W4A4_OK)
        return st;
    if (M == 0 || N == 0)
        return quant_gemm(X, ldx, perm, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, nullptr, 0, stream,
                          NormArgs{nullptr, 0.0f, nullptr});
    if (w4a4_quant_gemm_workspace_bytes(M, N, K, n_out, group) > kScratchBytes)
        return W4A4_ERR_UNSUPPORTED;
    void *ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != W4A4_OK)
        return st;
    // the array keeps the last call's contents: the split-K arrival counters
    // at its start are cleared on the stream after the argument checks and
    // before the launches (every other byte a call reads it has written first)
    return quant_gemm(X, ldx, perm, Wq4, Wq8, sw4, sw8, M, N, K, n_out, group, Y, ldy, ws, kScratchBytes, stream,
                      NormArgs{nullptr, 0.0f, nullptr}, true);
}

}  // extern "C"

