// Drives every host-side path of kda_abi.cpp (descriptor checks in order, pointer and
// workspace checks, workspace queries, the launch sequence with stand-in launchers)
// under AddressSanitizer / UndefinedBehaviorSanitizer.  Prints "abi driver ok" and
// exits 0 when every status is the expected one.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/kda.h"

extern int g_stub_launches;

static int failures = 0;
#define EXPECT(cond, what)                                                        \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::printf("FAIL %s (line %d)\n", what, __LINE__);                  \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static kda_fwd_desc base() {
    kda_fwd_desc d;
    std::memset(&d, 0, sizeof(d));
    d.B = 1; d.T = 256; d.H = 2; d.HV = 4; d.K = 128; d.V = 128; d.chunk_size = 64; d.num_seqs = 1;
    d.qkv_dtype = KDA_DTYPE_BF16; d.g_dtype = KDA_DTYPE_BF16; d.beta_dtype = KDA_DTYPE_BF16;
    d.scale = 0.088f; d.lower_bound = -5.f;
    d.flags = KDA_GATE_IN_KERNEL | KDA_SAFE_GATE | KDA_HAS_LOWER_BOUND | KDA_QK_L2NORM | KDA_BETA_SIGMOID |
              KDA_OUTPUT_FINAL_STATE;
    return d;
}

int main() {
    // fake device pointers: never dereferenced on the host
    char fake_buf[256];
    void *F = fake_buf;
    float *Ff = reinterpret_cast<float *>(fake_buf);
    size_t ws = 0;

    kda_fwd_desc d = base();
    EXPECT(kda_chunk_fwd_workspace_size(&d, &ws) == KDA_OK && ws > 0, "valid workspace query");
    EXPECT(kda_chunk_fwd_workspace_size(&d, nullptr) == KDA_ERR_NULL_POINTER, "null bytes pointer");
    EXPECT(kda_chunk_fwd_workspace_size(nullptr, &ws) == KDA_ERR_NULL_POINTER, "null descriptor");

    struct Case { const char *what; void (*edit)(kda_fwd_desc &); kda_status want; };
    const Case cases[] = {
        {"chunk 48", [](kda_fwd_desc &x) { x.chunk_size = 48; }, KDA_ERR_CHUNK_SIZE},
        {"K 512", [](kda_fwd_desc &x) { x.K = 512; x.V = 512; }, KDA_ERR_HEAD_DIM},
        {"K 80", [](kda_fwd_desc &x) { x.K = 80; }, KDA_ERR_UNSUPPORTED},
        {"V 48", [](kda_fwd_desc &x) { x.V = 48; }, KDA_ERR_UNSUPPORTED},
        {"V 288", [](kda_fwd_desc &x) { x.V = 288; }, KDA_ERR_UNSUPPORTED},
        {"fp32 K=V=256", [](kda_fwd_desc &x) { x.K = 256; x.V = 256; x.qkv_dtype = KDA_DTYPE_FP32; }, KDA_ERR_UNSUPPORTED},
        {"GVA", [](kda_fwd_desc &x) { x.H = 3; }, KDA_ERR_GVA},
        {"lb -6", [](kda_fwd_desc &x) { x.lower_bound = -6.f; }, KDA_ERR_LOWER_BOUND},
        {"lb NaN", [](kda_fwd_desc &x) { x.lower_bound = NAN; }, KDA_ERR_LOWER_BOUND},
        {"neg eigval", [](kda_fwd_desc &x) { x.flags = KDA_ALLOW_NEG_EIGVAL; }, KDA_ERR_NEG_EIGVAL},
        {"dtype", [](kda_fwd_desc &x) { x.g_dtype = 9; }, KDA_ERR_DTYPE},
        {"T < 0", [](kda_fwd_desc &x) { x.T = -1; }, KDA_ERR_SHAPE},
        {"B*T overflow", [](kda_fwd_desc &x) { x.B = 1 << 20; x.T = 1 << 20; x.num_seqs = 1 << 20; }, KDA_ERR_SHAPE},
        {"flag bit", [](kda_fwd_desc &x) { x.flags |= 1u << 20; }, KDA_ERR_UNSUPPORTED},
    };
    for (const Case &c : cases) {
        kda_fwd_desc x = base();
        c.edit(x);
        EXPECT(kda_chunk_fwd_workspace_size(&x, &ws) == c.want, c.what);
        EXPECT(kda_chunk_fwd(&x, F, F, F, F, F, Ff, nullptr, nullptr, nullptr, F, Ff, F, size_t(1) << 40, nullptr) == c.want,
               c.what);
    }

    // varlen plans: valid, empty segment, bad offsets
    const int64_t cu_ok[4] = {0, 100, 100, 256};
    const int64_t cu_bad[4] = {0, 120, 100, 256};
    d = base();
    d.num_seqs = 3;
    d.cu_seqlens_host = cu_ok;
    EXPECT(kda_chunk_fwd_workspace_size(&d, &ws) == KDA_OK, "varlen query");
    d.cu_seqlens_host = cu_bad;
    EXPECT(kda_chunk_fwd_workspace_size(&d, &ws) == KDA_ERR_VARLEN, "decreasing offsets");

    // pointer and workspace checks, then a full launch sequence through the stand-ins
    d = base();
    EXPECT(kda_chunk_fwd_workspace_size(&d, &ws) == KDA_OK, "query");
    EXPECT(kda_chunk_fwd(&d, nullptr, F, F, F, F, Ff, nullptr, nullptr, nullptr, F, Ff, F, ws, nullptr) ==
               KDA_ERR_NULL_POINTER, "null q");
    EXPECT(kda_chunk_fwd(&d, F, F, F, F, F, Ff, nullptr, nullptr, nullptr, F, nullptr, F, ws, nullptr) ==
               KDA_ERR_NULL_POINTER, "null final_state");
    EXPECT(kda_chunk_fwd(&d, F, F, F, F, F, Ff, nullptr, nullptr, nullptr, F, Ff, F, ws - 1, nullptr) ==
               KDA_ERR_WORKSPACE, "short workspace");
    const int before = g_stub_launches;
    EXPECT(kda_chunk_fwd(&d, F, F, F, F, F, Ff, nullptr, nullptr, nullptr, F, Ff, F, ws, nullptr) == KDA_OK,
           "launch sequence");
    EXPECT(g_stub_launches > before, "stages launched");

    // gate entry and backward entry: queries and checks
    size_t gws = 0, bws = 0;
    EXPECT(kda_gate_chunk_cumsum_workspace_size(&d, &gws) == KDA_OK, "gate query");
    EXPECT(kda_gate_chunk_cumsum(&d, F, Ff, nullptr, nullptr, nullptr, Ff, F, gws, nullptr) == KDA_OK, "gate launch");
    EXPECT(kda_chunk_bwd_workspace_size(&d, &bws) == KDA_OK && bws >= ws, "bwd query");
    kda_fwd_desc t = base();
    t.flags |= KDA_TRANSPOSE_STATE;
    EXPECT(kda_chunk_bwd_workspace_size(&t, &bws) == KDA_ERR_UNSUPPORTED, "bwd transposed state");

    for (int s = 0; s <= KDA_ERR_HIP + 1; ++s) EXPECT(kda_status_string((kda_status)s) != nullptr, "status string");
    EXPECT(kda_abi_version() == KDA_ABI_VERSION, "abi version");

    if (failures == 0) std::printf("abi driver ok\n");
    return failures == 0 ? 0 : 1;
}
