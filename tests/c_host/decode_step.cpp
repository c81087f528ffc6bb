// One decode step through the C ABI from a plain C++ host program (no Python,
// no torch in the process): index score with gate bits -> compaction from the
// bits -> top-k -> sparse attention, on buffers this program allocates.
//
// usage: decode_step <in.bin> <out.bin>
// in.bin (little-endian): int32 B, S_max, H, D, k, Hq, Dl, max_hca; float bias,
// scale; then int32 seq_len[B], int32 hca_count[B]; bf16 keys [sum S, D],
// q [B, H, D]; fp32 w [B, H]; bf16 qa [B, Hq, Dl], latent [sum S, Dl],
// hca [sum hca, Dl].  Sequences are packed (entry, key and latent row starts
// are the running sums of seq_len, HCA row starts those of hca_count).
// out.bin: fp32 z [sum S]; int32 cand_count [B], cand_idx [sum S]; int32
// topk_count [B], topk_idx [B, k]; bf16 out [B, Hq, Dl]; fp32 lse [B, Hq].
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "lsa.h"

#define CHECK_HIP(x)                                                            \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));        \
            std::exit(2);                                                       \
        }                                                                       \
    } while (0)
#define CHECK_LSA(x)                                                            \
    do {                                                                        \
        int s_ = (x);                                                           \
        if (s_ != LSA_OK) {                                                     \
            std::fprintf(stderr, "%s: %s (%s)\n", #x, lsa_status_string(s_),    \
                         lsa_last_error());                                     \
            std::exit(3);                                                       \
        }                                                                       \
    } while (0)

template <typename T>
static std::vector<T> read_vec(std::FILE* f, size_t n) {
    std::vector<T> v(n);
    if (n && std::fread(v.data(), sizeof(T), n, f) != n) {
        std::fprintf(stderr, "short input file\n");
        std::exit(4);
    }
    return v;
}

template <typename T>
static T* to_device(const std::vector<T>& v) {
    T* p = nullptr;
    CHECK_HIP(hipMalloc(&p, v.empty() ? 16 : v.size() * sizeof(T)));
    if (!v.empty()) CHECK_HIP(hipMemcpy(p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice));
    return p;
}

template <typename T>
static T* device_buffer(size_t n) {
    T* p = nullptr;
    CHECK_HIP(hipMalloc(&p, (n ? n : 1) * sizeof(T)));
    return p;
}

template <typename T>
static void write_back(std::FILE* f, const T* d, size_t n) {
    std::vector<T> h(n);
    if (n) CHECK_HIP(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    std::fwrite(h.data(), sizeof(T), n, f);
}

int main(int argc, char** argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
        return 1;
    }
    std::FILE* fi = std::fopen(argv[1], "rb");
    if (!fi) return 1;
    const auto hdr = read_vec<int32_t>(fi, 8);
    const int B = hdr[0], S_max = hdr[1], H = hdr[2], D = hdr[3], k = hdr[4], Hq = hdr[5],
              Dl = hdr[6], max_hca = hdr[7];
    const auto fp = read_vec<float>(fi, 2);
    const float bias = fp[0], scale = fp[1];
    const auto seq_len = read_vec<int32_t>(fi, B);
    const auto hca_count = read_vec<int32_t>(fi, B);
    std::vector<int64_t> starts(B), hca_starts(B);
    int64_t total = 0, total_hca = 0;
    for (int b = 0; b < B; ++b) {
        starts[b] = total;
        hca_starts[b] = total_hca;
        total += seq_len[b];
        total_hca += hca_count[b];
    }
    const auto keys = read_vec<uint16_t>(fi, (size_t)total * D);
    const auto q = read_vec<uint16_t>(fi, (size_t)B * H * D);
    const auto w = read_vec<float>(fi, (size_t)B * H);
    const auto qa = read_vec<uint16_t>(fi, (size_t)B * Hq * Dl);
    const auto latent = read_vec<uint16_t>(fi, (size_t)total * Dl);
    const auto hca = read_vec<uint16_t>(fi, (size_t)total_hca * Dl);
    std::fclose(fi);

    int32_t* d_len = to_device(seq_len);
    int64_t* d_start = to_device(starts);
    int32_t* d_hcnt = to_device(hca_count);
    int64_t* d_hstart = to_device(hca_starts);
    uint16_t* d_keys = to_device(keys);
    uint16_t* d_q = to_device(q);
    float* d_w = to_device(w);
    uint16_t* d_qa = to_device(qa);
    uint16_t* d_lat = to_device(latent);
    uint16_t* d_hca = to_device(hca);
    float* d_z = device_buffer<float>(total);
    uint16_t* d_gate = device_buffer<uint16_t>((size_t)B * lsa_gate_words(S_max));
    int32_t* d_cand = device_buffer<int32_t>(total);
    int32_t* d_ccnt = device_buffer<int32_t>(B);
    int32_t* d_tk = device_buffer<int32_t>((size_t)B * k);
    int32_t* d_tcnt = device_buffer<int32_t>(B);
    uint16_t* d_out = device_buffer<uint16_t>((size_t)B * Hq * Dl);
    float* d_lse = device_buffer<float>((size_t)B * Hq);
    CHECK_HIP(hipMemset(d_tk, 0xff, (size_t)B * k * sizeof(int32_t)));
    const size_t ws_t = lsa_workspace_bytes(LSA_OP_TOPK, B, 0, 0, 0, S_max, k, 0);
    const size_t ws_a = lsa_workspace_bytes(LSA_OP_ATTEND, B, 1, Hq, Dl, 0, k, max_hca);
    void* d_ws_t = device_buffer<unsigned char>(ws_t);
    void* d_ws_a = device_buffer<unsigned char>(ws_a);

    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    CHECK_LSA(lsa_index_score(d_keys, LSA_DTYPE_BF16, d_start, d_len, d_start, B, 1, H, D, S_max,
                              d_q, d_w, bias, 1, d_z, nullptr, d_gate, 0.0f, st));
    CHECK_LSA(lsa_select_compact(nullptr, d_gate, d_start, d_len, B, S_max, 0.0f, d_cand, d_ccnt,
                                 nullptr, 0, st));
    CHECK_LSA(lsa_topk(d_z, d_start, d_len, B, S_max, d_cand, d_ccnt, k, d_tk, d_tcnt, 0, d_ws_t,
                       ws_t, st));
    CHECK_LSA(lsa_sparse_attend(d_qa, LSA_DTYPE_BF16, B, 1, Hq, Dl, d_lat, d_start, d_tk, d_tcnt,
                                k, total_hca ? d_hca : nullptr, d_hstart, d_hcnt, max_hca, scale,
                                d_out, d_lse, d_ws_a, ws_a, st));
    CHECK_HIP(hipStreamSynchronize(st));

    std::FILE* fo = std::fopen(argv[2], "wb");
    if (!fo) return 1;
    write_back(fo, d_z, total);
    write_back(fo, d_ccnt, B);
    write_back(fo, d_cand, total);
    write_back(fo, d_tcnt, B);
    write_back(fo, d_tk, (size_t)B * k);
    write_back(fo, d_out, (size_t)B * Hq * Dl);
    write_back(fo, d_lse, (size_t)B * Hq);
    std::fclose(fo);
    CHECK_HIP(hipStreamDestroy(st));
    std::printf("decode step ok\n");
    return 0;
}
