// Exercises libtg's host code -- argument validation, the dispatcher's plans,
// the configuration table, the tuning-cache parser and the attention
// argument checks -- under AddressSanitizer and UndefinedBehaviorSanitizer,
// on a machine without a GPU: device pointers are stand-in addresses that no
// call dereferences (every call that would launch stops at the device check).
// Exits 0 when every call returned an allowed status and the plan invariants
// held.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <thread>
#include <vector>

#include "tg.h"
#include "tg_diag.h"

static int failures;
#define EXPECT(c)                                                                      \
    do {                                                                               \
        if (!(c)) {                                                                    \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c);           \
            failures++;                                                                \
        }                                                                              \
    } while (0)

static uint64_t rng = 0x243f6a8885a308d3ull;
static uint64_t next()
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return rng;
}
static int64_t pick(const int64_t *v, int n) { return v[next() % (uint64_t)n]; }

static const void *at(uintptr_t a) { return reinterpret_cast<const void *>(a); }

// Plans on random shapes, layouts, alignments and workspace sizes: the call
// validates, the plan's configuration can run the problem (or its packed
// copies), and the workspace it uses fits.
static void plans()
{
    const int64_t dims[] = {0, 1, 2, 15, 16, 17, 64, 127, 256, 257, 1000, 1031, 3001, 4096, 8192};
    const size_t wss[] = {0, 16, 1 << 20, (size_t)64 << 20, (size_t)1 << 40, SIZE_MAX};
    const int n = tg_num_configs();
    for (int it = 0; it < 4000; it++) {
        const int64_t M = pick(dims, 15), N = pick(dims, 15), K = pick(dims, 15);
        const tg_op oa = (tg_op)(next() & 1), ob = (tg_op)(next() & 1);
        const tg_dtype dt = (tg_dtype)(1 + next() % 3);
        const int es = dt == TG_DTYPE_I32 ? 1 : 2;
        const int64_t lda = (oa ? M : K) + (int64_t)(next() % 3) * (int64_t)(next() % 9);
        const int64_t ldb = (ob ? K : N) + (int64_t)(next() % 3) * (int64_t)(next() % 9);
        const int64_t ldc = N + (int64_t)(next() % 2) * 8;
        const uintptr_t A = 0x1000000 + (uintptr_t)(es * (next() % 3) * (next() % 2));
        const uintptr_t B = 0x9000000 + (uintptr_t)(es * (next() % 3) * (next() % 2));
        const float *bias = (dt != TG_DTYPE_I32 && (next() & 1)) ? (const float *)at(0x11000000) : nullptr;
        const size_t ws = wss[next() % 6];
        int cid = -7, sp = -7, packed = -7;
        size_t used = 7;
        const tg_status st = tg_select_plan(oa, ob, at(A), at(B), bias, at(0x20000000), M, N, K,
                                            lda, ldb, ldc, dt, ws, &cid, &sp, &packed, &used);
        EXPECT(st == TG_SUCCESS || st == TG_ERROR_INVALID_VALUE || st == TG_ERROR_UNSUPPORTED);
        if (st != TG_SUCCESS)
            continue;
        EXPECT(used <= ws);
        if (M == 0 || N == 0) {
            EXPECT(cid == -1 && sp == 1 && packed == 0 && used == 0);
            continue;
        }
        EXPECT(cid >= 0 && cid < n && sp >= 1 && sp <= 64 && packed >= 0 && packed <= 3);
        if (packed == 0)
            EXPECT(tg_config_supports(cid, oa, ob, at(A), at(B), bias, at(0x20000000), M, N, K,
                                      lda, ldb, ldc, dt) == 1);
        if (sp > 1)
            EXPECT(used >= tg_splitk_workspace_bytes(M, N, sp));
        const int plain = tg_select_config(oa, ob, at(A), at(B), bias, at(0x20000000), M, N, K,
                                           lda, ldb, ldc, dt);
        EXPECT(plain >= 0 && plain < n);
        // every call stops at the device check (no GPU here) or earlier
        const tg_status g = tg_gemm_ws(-1, 0, oa, ob, at(A), at(B), bias, (void *)at(0x20000000),
                                       M, N, K, lda, ldb, ldc, dt, (void *)at(0x30000000), ws,
                                       nullptr);
        EXPECT(g != TG_SUCCESS && g != TG_ERROR_LAUNCH);
    }
}

static void invalid_arguments()
{
    void *P = (void *)at(0x100000);
    EXPECT(tg_gemm(P, P, P, -1, 4, 4, 4, 4, 4, TG_DTYPE_F32, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm(P, P, P, 4, 4, 4, 3, 4, 4, TG_DTYPE_F32, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm(P, P, P, 4, 4, 4, 4, 4, 4, (tg_dtype)9, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm(nullptr, P, P, 4, 4, 4, 4, 4, 4, TG_DTYPE_F32, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm(P, P, P, 0, 4, 4, 4, 4, 4, TG_DTYPE_F32, nullptr) == TG_SUCCESS);
    EXPECT(tg_gemm(P, P, P, (int64_t)1 << 40, 4, 4, 4, 4, 4, TG_DTYPE_F32, nullptr) ==
           TG_ERROR_UNSUPPORTED);
    EXPECT(tg_gemm_bias_relu(P, P, nullptr, P, 4, 4, 4, 4, 4, 4, TG_DTYPE_F16, nullptr) ==
           TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ex((tg_op)2, TG_OP_N, P, P, nullptr, P, 4, 4, 4, 4, 4, 4, TG_DTYPE_F32,
                      nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_with_config(tg_num_configs(), TG_OP_N, TG_OP_N, P, P, nullptr, P, 4, 4, 4, 4,
                               4, 4, TG_DTYPE_F32, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ws(-1, 65, TG_OP_N, TG_OP_N, P, P, nullptr, P, 4, 4, 4, 4, 4, 4, TG_DTYPE_F32,
                      P, 1 << 20, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ws(-1, 4, TG_OP_N, TG_OP_N, P, P, nullptr, P, 640, 640, 8192, 8192, 640, 640,
                      TG_DTYPE_F32, P, 16, nullptr) == TG_ERROR_WORKSPACE);
    EXPECT(tg_gemm_ws(-1, 4, TG_OP_N, TG_OP_N, P, P, nullptr, P, 640, 640, 8192, 8192, 640, 640,
                      TG_DTYPE_F32, nullptr, 16, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_gemm_ws_static(-1, 4, TG_OP_N, TG_OP_N, P, P, nullptr, P, 640, 640, 8192, 8192,
                             640, 640, TG_DTYPE_F32, nullptr) != TG_SUCCESS);
    int cid, sp, pk;
    size_t used;
    EXPECT(tg_select_plan(TG_OP_N, TG_OP_N, P, P, nullptr, P, 4, 4, 4, 4, 4, 4, TG_DTYPE_F32, 0,
                          &cid, nullptr, &pk, &used) == TG_ERROR_INVALID_VALUE);
    tg_config_desc d;
    for (int i = 0; i < tg_num_configs(); i++) {
        EXPECT(tg_config_info(i, &d) == TG_SUCCESS && d.id == i && d.name && strlen(d.name) > 4);
        for (int op = 0; op < 4; op++)
            EXPECT(tg_config_supports(i, (tg_op)(op >> 1), (tg_op)(op & 1), P, P, nullptr, P, 100,
                                      100, 100, 100, 100, 100, TG_DTYPE_F16) >= 0);
    }
    EXPECT(tg_config_info(-1, &d) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_config_info(0, nullptr) == TG_ERROR_INVALID_VALUE);
    for (int s = -1; s < 9; s++)
        EXPECT(tg_status_string((tg_status)s) != nullptr);
    EXPECT(strstr(tg_version(), "gfx950") != nullptr);
    EXPECT(tg_splitk_workspace_bytes(640, 640, 8) == (size_t)8 * 640 * 640 * 4);
    EXPECT(tg_splitk_workspace_bytes(640, 640, 65) == 0);
    // the ceiling's arguments
    float *sink = (float *)at(0x200000);
    EXPECT(tg_mfma_ceiling(8, P, sink, 2, 1, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_mfma_ceiling(32, P, sink, 3, 1, nullptr) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_mfma_ceiling(32, P, sink, (int64_t)1 << 30, (int64_t)1 << 20, nullptr) ==
           TG_ERROR_INVALID_VALUE);
}

static void attention_arguments()
{
    const void *P = at(0x100000);
    const int64_t s[3] = {16 * 4096 * 128, 4096 * 128, 128}, neg[3] = {1, -8, 8};
    const struct {
        int64_t B, H, Hkv, Lq, Lk, d;
        const int64_t *st;
        float scale;
        int causal;
        tg_status want;
    } cases[] = {
        {-1, 16, 16, 64, 64, 128, s, 0.1f, 0, TG_ERROR_INVALID_VALUE},
        {1, 16, 5, 64, 64, 128, s, 0.1f, 0, TG_ERROR_INVALID_VALUE},
        {1, 16, 16, 64, 64, 128, neg, 0.1f, 0, TG_ERROR_INVALID_VALUE},
        {1, 16, 16, 64, 64, 128, s, __builtin_nanf(""), 0, TG_ERROR_INVALID_VALUE},
        {1, 16, 16, 64, 64, 128, s, 0.1f, 2, TG_ERROR_INVALID_VALUE},
        {1, 16, 16, 64, 64, 96, s, 0.1f, 0, TG_ERROR_UNSUPPORTED},
        {0, 16, 16, 64, 64, 128, s, 0.1f, 0, TG_SUCCESS},
        {1, 16, 16, 0, 64, 128, s, 0.1f, 1, TG_SUCCESS},
    };
    for (const auto &c : cases)
        EXPECT(tg_attention_fwd(P, P, P, (void *)P, nullptr, c.B, c.H, c.Hkv, c.Lq, c.Lk, c.d,
                                c.st, c.st, c.st, c.st, c.scale, c.causal, nullptr) == c.want);
    EXPECT(tg_attention_fwd(P, P, P, (void *)P, nullptr, 1, 16, 16, 64, 64, 128, nullptr, s, s, s,
                            0.1f, 0, nullptr) == TG_ERROR_INVALID_VALUE);
}

// Tuning-cache files: well-formed, stale, malformed and over-long records,
// loaded while other threads plan against the cache.
static void tuning(const char *dir)
{
    tg_config_desc d;
    tg_config_info(3, &d);
    const std::string name = d.name;
    const std::string path = std::string(dir) + "/t.tgtune";
    auto write = [&](const std::string &text) {
        FILE *f = fopen(path.c_str(), "w");
        if (f == nullptr) {
            fprintf(stderr, "cannot write %s\n", path.c_str());
            exit(2);
        }
        fputs(text.c_str(), f);
        fclose(f);
    };
    int loaded = -1, skipped = -1, line = -1;
    write("tg-tuning 1\n# comment\n\n512 512 512 N N f16 0 3 " + name + " 100.5\n"
          "640 640 640 T N f32 1 3 " + name + " 1\n"
          "64 64 64 N N f16 0 3 not_this_name 1\n"
          "64 64 64 N N i32 0 99999 x 1\n");
    EXPECT(tg_tuning_load(path.c_str(), &loaded, &skipped, &line) == TG_SUCCESS);
    EXPECT(loaded == 2 && skipped == 2 && tg_tuning_count() == 2);
    const char *bad[] = {"tg-tuning 2\n", "", "tg-tuning 1\n1 2 3\n",
                         "tg-tuning 1\n1 2 3 N N f16 0 3 x 1 extra\n",
                         "tg-tuning 1\n1 2 3 Q N f16 0 3 x 1\n",
                         "tg-tuning 1\n1 2 3 N N f16 2 3 x 1\n",
                         "tg-tuning 1\n1 2 3 N N i32 1 3 x 1\n",
                         "tg-tuning 1\n-1 2 3 N N f16 0 3 x 1\n",
                         "tg-tuning 1\n1 2 3 N N f16 0 3 x nan\n",
                         "tg-tuning 1\n99999999999999999999 2 3 N N f16 0 3 x 1\n"};
    for (const char *b : bad) {
        write(b);
        EXPECT(tg_tuning_load(path.c_str(), &loaded, &skipped, &line) == TG_ERROR_INVALID_VALUE);
        EXPECT(tg_tuning_count() == 2);   // unchanged by a failed load
    }
    write("tg-tuning 1\n" + std::string(5000, '7') + "\n");
    EXPECT(tg_tuning_load(path.c_str(), nullptr, nullptr, &line) == TG_ERROR_INVALID_VALUE);
    EXPECT(tg_tuning_load((std::string(dir) + "/missing").c_str(), nullptr, nullptr, &line) ==
           TG_ERROR_FILE);
    EXPECT(tg_tuning_load(nullptr, nullptr, nullptr, &line) == TG_ERROR_INVALID_VALUE);
    // many records, reloaded while four threads plan against the cache
    std::string big = "tg-tuning 1\n";
    for (int i = 1; i <= 3000; i++)
        big += std::to_string(16 * i) + " 512 512 N N f16 0 3 " + name + " 1\n";
    write(big);
    std::vector<std::thread> th;
    for (int t = 0; t < 4; t++)
        th.emplace_back([t] {
            for (int i = 0; i < 3000; i++) {
                int cid, sp, pk;
                size_t used;
                const int64_t M = 16 * (1 + (i * 7 + t) % 3000);
                if (tg_select_plan(TG_OP_N, TG_OP_N, at(0x100000), at(0x200000), nullptr,
                                   at(0x300000), M, 512, 512, 512, 512, 512, TG_DTYPE_F16,
                                   SIZE_MAX, &cid, &sp, &pk, &used) != TG_SUCCESS)
                    __atomic_add_fetch(&failures, 1, __ATOMIC_RELAXED);
            }
        });
    for (int r = 0; r < 20; r++) {
        EXPECT(tg_tuning_load(path.c_str(), &loaded, nullptr, nullptr) == TG_SUCCESS);
        EXPECT(loaded == 3000);
        tg_tuning_clear();
    }
    for (auto &t : th)
        t.join();
    EXPECT(tg_tuning_load(path.c_str(), &loaded, nullptr, nullptr) == TG_SUCCESS);
    int cid, sp, pk;
    size_t used;
    EXPECT(tg_select_plan(TG_OP_N, TG_OP_N, at(0x100000), at(0x200000), nullptr, at(0x300000), 1600,
                          512, 512, 512, 512, 512, TG_DTYPE_F16, SIZE_MAX, &cid, &sp, &pk,
                          &used) == TG_SUCCESS &&
           cid == 3 && sp == 1);
    tg_tuning_clear();
    EXPECT(tg_tuning_count() == 0);
}

int main(int argc, char **argv)
{
    // the configuration table as this build sees it, for comparison with
    // the library's
    tg_config_desc d;
    for (int i = 0; i < tg_num_configs(); i++)
        if (tg_config_info(i, &d) == TG_SUCCESS)
            printf("config %d %d %d %d %d %d %d %d %d %d %d %d %d %s\n", d.id, d.block_m,
                   d.block_n, d.block_k, d.stages, d.waves_m, d.waves_n, d.mfma, d.direct_lds,
                   d.lds_bytes, d.ops, d.elem_bytes, d.whole_k, d.name);
    invalid_arguments();
    attention_arguments();
    plans();
    tuning(argc > 1 ? argv[1] : ".");
    if (failures)
        fprintf(stderr, "%d failures\n", failures);
    else
        printf("host driver ok\n");
    return failures ? 1 : 0;
}
