/*
 * The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on
 * the host alone (tests/test_abi_asan.py builds it with stub launchers).
 *
 * Every "device" pointer points into a PROT_NONE mapping, so the host layer
 * faults if it ever reads or writes caller memory itself.  Calls with
 * invalid arguments must be refused before any launch (the stubs count the
 * calls that get past their checks); valid calls must reach a launch (which
 * the stubs fail, so they return SA_ERR_HIP).  A sweep of dims through the
 * split table and the workspace sizing runs the planner's arithmetic over
 * extreme sizes.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <sys/mman.h>

#include "sa.h"

int sa_test_launch_count(void);

static int g_checks = 0, g_fail = 0;
#define CHECK(cond, ...)                                        \
    do {                                                        \
        ++g_checks;                                             \
        if (!(cond)) {                                          \
            ++g_fail;                                           \
            fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                       \
            fprintf(stderr, "\n");                              \
        }                                                       \
    } while (0)

static char* g_dev;   /* a PROT_NONE region standing for device memory */
#define DEV(off) ((void*)(g_dev + (off)))

static sa_dims good(void) {
    sa_dims d;
    memset(&d, 0, sizeof d);
    d.num_seqs = 4;
    d.num_q_heads = 32;
    d.num_kv_heads = 4;
    d.head_dim = 64;
    d.block_size = 16;
    d.max_blocks_per_seq = 64;   /* 1024 slots: the table splits it, so a workspace */
    d.num_blocks = 256;
    d.cache_layout = SA_LAYOUT_K2_V8;
    return d;
}

/* one call of every entry point that takes pools, on dims d and the window;
   which = index of a pointer argument to make NULL (-1: none), mis = the
   same to make misaligned */
typedef int (*call_fn)(const sa_dims* d, int32_t w, int which, int mis, size_t ws_bytes);

static void* ptr(int i, int which, int mis) {
    if (i == which) return NULL;
    return (char*)DEV((size_t)i << 16) + (i == mis ? 2 : 0);
}

static int call_append(const sa_dims* d, int32_t w, int which, int mis, size_t ws) {
    (void)ws;
    return sa_kv_append(ptr(0, which, mis), ptr(1, which, mis), ptr(2, which, mis),
                        ptr(3, which, mis), ptr(4, which, mis), ptr(5, which, mis), w, d, NULL);
}
static int call_attention(const sa_dims* d, int32_t w, int which, int mis, size_t ws) {
    return sa_decode_attention(ptr(0, which, mis), ptr(1, which, mis), ptr(2, which, mis),
                               ptr(3, which, mis), ptr(4, which, mis), ptr(5, -1, -1), w,
                               ptr(6, which, mis), d, ws ? ptr(7, which, mis) : NULL, ws, NULL);
}
static int call_fused(const sa_dims* d, int32_t w, int which, int mis, size_t ws) {
    return sa_decode_attention_append(ptr(0, which, mis), ptr(1, which, mis), ptr(2, which, mis),
                                      ptr(3, which, mis), ptr(4, which, mis), ptr(5, which, mis),
                                      ptr(6, which, mis), ptr(7, -1, -1), w, ptr(8, which, mis),
                                      d, ws ? ptr(9, which, mis) : NULL, ws, NULL);
}
static int call_noalloc(const sa_dims* d, int32_t w, int which, int mis, size_t ws) {
    (void)ws;
    return sa_decode_attention_append_noalloc(ptr(0, which, mis), ptr(1, which, mis),
                                              ptr(2, which, mis), ptr(3, which, mis),
                                              ptr(4, which, mis), ptr(5, which, mis),
                                              ptr(6, which, mis), ptr(7, -1, -1), w,
                                              ptr(8, which, mis), d, NULL);
}
static int call_rope(const sa_dims* d, int32_t w, int which, int mis, size_t ws) {
    sa_rope r = {(const float*)ptr(10, which, mis), (const float*)ptr(11, which, mis), 4096,
                 SA_ROPE_HALF};
    return sa_decode_attention_append_rope(ptr(0, which, mis), ptr(1, which, mis),
                                           ptr(2, which, mis), ptr(3, which, mis),
                                           ptr(4, which, mis), ptr(5, which, mis),
                                           ptr(6, which, mis), ptr(7, -1, -1), w, &r,
                                           ptr(8, which, mis), d,
                                           ws ? ptr(9, which, mis) : NULL, ws, NULL);
}
static int call_partials(const sa_dims* d, int32_t w, int which, int mis, size_t ws) {
    (void)ws;
    return sa_decode_partials(ptr(0, which, mis), ptr(1, which, mis), ptr(2, which, mis),
                              ptr(3, which, mis), ptr(4, which, mis), w, ptr(5, which, mis),
                              ptr(6, which, mis), d, NULL);
}

/* nptr pointer arguments; sinks_idx: the one a caller may leave NULL (-1: none) */
static const struct { const char* name; call_fn f; int nptr; int uses_ws; int sinks_idx; } CALLS[] = {
    {"kv_append", call_append, 6, 0, -1},
    {"decode_attention", call_attention, 8, 1, 5},
    {"decode_attention_append", call_fused, 10, 1, 7},
    {"noalloc", call_noalloc, 9, 0, 7},
    {"rope", call_rope, 12, 1, 7},
    {"partials", call_partials, 7, 0, -1},
};
#define NCALLS ((int)(sizeof CALLS / sizeof CALLS[0]))

/* refused before any launch */
static void expect_refused(const char* what, int st, int before) {
    CHECK(st < 0 && st != SA_ERR_HIP && sa_test_launch_count() == before,
          "%s: status %d, launches %d -> %d (want a refusal before any launch)", what, st, before,
          sa_test_launch_count());
}
/* got past its checks to a launch */
static void expect_launched(const char* what, int st, int before) {
    CHECK(st == SA_ERR_HIP && sa_test_launch_count() > before,
          "%s: status %d, launches %d -> %d (want a launch, failed by the stub)", what, st, before,
          sa_test_launch_count());
}

static void entry_points(void) {
    const sa_dims d0 = good();
    for (int c = 0; c < NCALLS; ++c) {
        const size_t ws = CALLS[c].uses_ws ? sa_decode_workspace_bytes(&d0, 0) : 0;
        int before = sa_test_launch_count();
        expect_launched(CALLS[c].name, CALLS[c].f(&d0, 0, -1, -1, ws), before);
        /* NULL dims */
        before = sa_test_launch_count();
        expect_refused(CALLS[c].name, CALLS[c].f(NULL, 0, -1, -1, ws), before);
        /* each pointer NULL, then each misaligned */
        for (int i = 0; i < CALLS[c].nptr; ++i) {
            if (i == CALLS[c].sinks_idx) continue;        /* sinks may be NULL */
            char what[96];
            snprintf(what, sizeof what, "%s NULL pointer %d", CALLS[c].name, i);
            before = sa_test_launch_count();
            const int st = CALLS[c].f(&d0, 0, i, -1, ws);
            /* a NULL workspace for a call that needs one, or NULL pointers */
            expect_refused(what, st, before);
        }
        /* num_seqs = 0: nothing to do, nothing launched */
        sa_dims d = d0;
        d.num_seqs = 0;
        before = sa_test_launch_count();
        const int st0 = CALLS[c].f(&d, 0, -1, -1, ws);
        CHECK(st0 == SA_OK && sa_test_launch_count() == before, "%s: B = 0 gave %d",
              CALLS[c].name, st0);
        /* bad dims, each refused */
        sa_dims bad[16];
        int nb = 0;
        bad[nb] = d0; bad[nb++].num_seqs = -1;
        bad[nb] = d0; bad[nb++].num_q_heads = 0;
        bad[nb] = d0; bad[nb++].num_kv_heads = 0;
        bad[nb] = d0; bad[nb++].num_q_heads = 30;               /* not a multiple of Hkv */
        bad[nb] = d0; bad[nb++].head_dim = 128;
        bad[nb] = d0; bad[nb++].block_size = 12;
        bad[nb] = d0; bad[nb++].block_size = 128;
        bad[nb] = d0; bad[nb++].max_blocks_per_seq = 0;
        bad[nb] = d0; bad[nb++].max_blocks_per_seq = INT32_MAX; /* capacity past 2^30 */
        bad[nb] = d0; bad[nb++].num_blocks = -5;
        bad[nb] = d0; bad[nb++].variant = 6;
        bad[nb] = d0; bad[nb++].variant = -1;
        bad[nb] = d0; bad[nb++].cache_layout = SA_LAYOUT_PLAIN;
        bad[nb] = d0; bad[nb++].cache_layout = 7;
        bad[nb] = d0; bad[nb++].num_query_tokens = 5;           /* 5 x 8 columns > 16 */
        bad[nb] = d0; bad[nb++].num_splits = -2;
        for (int j = 0; j < nb; ++j) {
            char what[96];
            snprintf(what, sizeof what, "%s bad dims #%d", CALLS[c].name, j);
            before = sa_test_launch_count();
            expect_refused(what, CALLS[c].f(&bad[j], 0, -1, -1, ws), before);
        }
        /* a window past the table's capacity */
        before = sa_test_launch_count();
        expect_refused("window past capacity", CALLS[c].f(&d0, 64 * 16 + 1, -1, -1, ws), before);
    }
    /* a workspace one byte short */
    {
        sa_dims d = good();
        d.num_splits = 4;
        const size_t need = sa_decode_workspace_bytes(&d, 0);
        CHECK(need > 0, "a split call needs a workspace");
        int before = sa_test_launch_count();
        expect_refused("short workspace", call_attention(&d, 0, -1, -1, need - 1), before);
        before = sa_test_launch_count();
        expect_refused("short workspace (fused)", call_fused(&d, 0, -1, -1, need - 1), before);
    }
    /* a query tile with a window is refused; without one it launches */
    {
        sa_dims d = good();
        d.num_query_tokens = 2;
        int before = sa_test_launch_count();
        expect_refused("tile with a window", call_fused(&d, 64, -1, -1, 1 << 24), before);
        before = sa_test_launch_count();
        expect_launched("tile", call_fused(&d, 0, -1, -1, sa_decode_workspace_bytes(&d, 0)),
                        before);
    }
    /* RoPE: NULL descriptor, bad style, no positions */
    {
        const sa_dims d = good();
        const size_t ws = sa_decode_workspace_bytes(&d, 0);
        sa_rope r = {(const float*)DEV(10 << 16), (const float*)DEV(11 << 16), 0, SA_ROPE_HALF};
        int before = sa_test_launch_count();
        expect_refused("rope NULL", sa_decode_attention_append_rope(
                           DEV(0), DEV(1 << 16), DEV(2 << 16), DEV(3 << 16), DEV(4 << 16),
                           DEV(5 << 16), DEV(6 << 16), NULL, 0, NULL, DEV(8 << 16), &d,
                           DEV(9 << 16), ws, NULL), before);
        before = sa_test_launch_count();
        expect_refused("rope no positions", sa_decode_attention_append_rope(
                           DEV(0), DEV(1 << 16), DEV(2 << 16), DEV(3 << 16), DEV(4 << 16),
                           DEV(5 << 16), DEV(6 << 16), NULL, 0, &r, DEV(8 << 16), &d,
                           DEV(9 << 16), ws, NULL), before);
        r.max_positions = 16;
        r.style = 9;
        before = sa_test_launch_count();
        expect_refused("rope bad style", sa_decode_attention_append_rope(
                           DEV(0), DEV(1 << 16), DEV(2 << 16), DEV(3 << 16), DEV(4 << 16),
                           DEV(5 << 16), DEV(6 << 16), NULL, 0, &r, DEV(8 << 16), &d,
                           DEV(9 << 16), ws, NULL), before);
    }
    /* combine */
    {
        const sa_dims d = good();
        int before = sa_test_launch_count();
        expect_launched("combine", sa_combine(DEV(0), DEV(1 << 16), NULL, 8, DEV(2 << 16), &d,
                                              NULL), before);
        before = sa_test_launch_count();
        expect_refused("combine S = 0", sa_combine(DEV(0), DEV(1 << 16), NULL, 0, DEV(2 << 16),
                                                   &d, NULL), before);
        before = sa_test_launch_count();
        expect_refused("combine NULL out", sa_combine(DEV(0), DEV(1 << 16), NULL, 8, NULL, &d,
                                                      NULL), before);
        before = sa_test_launch_count();
        expect_refused("combine NULL dims", sa_combine(DEV(0), DEV(1 << 16), NULL, 8,
                                                       DEV(2 << 16), NULL, NULL), before);
    }
    /* the probes */
    {
        int before = sa_test_launch_count();
        expect_launched("read probe", sa_read_bandwidth_probe(DEV(0), 4096, DEV(1 << 16), NULL),
                        before);
        before = sa_test_launch_count();
        expect_refused("read probe, 8 bytes", sa_read_bandwidth_probe(DEV(0), 8, DEV(1 << 16),
                                                                      NULL), before);
        before = sa_test_launch_count();
        expect_launched("tile probe", sa_read_tiles_probe(DEV(0), 1 << 20, DEV(1 << 16), 100, 64,
                                                          DEV(2 << 16), NULL), before);
        before = sa_test_launch_count();
        expect_refused("tile probe, 0 waves", sa_read_tiles_probe(DEV(0), 1 << 20, DEV(1 << 16),
                                                                  100, 0, DEV(2 << 16), NULL),
                       before);
        before = sa_test_launch_count();
        expect_refused("tile probe, -1 tiles", sa_read_tiles_probe(DEV(0), 1 << 20, DEV(1 << 16),
                                                                   -1, 64, DEV(2 << 16), NULL),
                       before);
    }
    /* status strings, known and unknown */
    for (int s = -7; s <= 1; ++s) CHECK(sa_status_string(s) != NULL, "status string %d", s);
}

/* The split table and workspace sizing over extreme dims; every valid
   configuration's call, given that workspace, reaches its launch. */
static void planner_sweep(void) {
    const int32_t Bs[] = {1, 2, 3, 64, 2047, 2048, 2049, 100000, INT32_MAX};
    const int32_t Hkvs[] = {1, 8, 64, 128};
    const int32_t Gs[] = {1, 8, 16};
    const int32_t bss[] = {8, 16, 32, 64};
    const int32_t mbss[] = {1, 7, 64, 8192, 1 << 20};
    const int32_t windows[] = {0, 1, 128, 1000};
    const int32_t Ts[] = {0, 2};
    int launched = 0;
    for (size_t a = 0; a < sizeof Bs / sizeof Bs[0]; ++a)
    for (size_t h = 0; h < sizeof Hkvs / sizeof Hkvs[0]; ++h)
    for (size_t g = 0; g < sizeof Gs / sizeof Gs[0]; ++g)
    for (size_t k = 0; k < sizeof bss / sizeof bss[0]; ++k)
    for (size_t m = 0; m < sizeof mbss / sizeof mbss[0]; ++m)
    for (size_t w = 0; w < sizeof windows / sizeof windows[0]; ++w)
    for (int v = 0; v <= 5; ++v)
    for (size_t t = 0; t < sizeof Ts / sizeof Ts[0]; ++t) {
        sa_dims d = good();
        d.num_seqs = Bs[a];
        d.num_kv_heads = Hkvs[h];
        d.num_q_heads = (int32_t)((int64_t)Hkvs[h] * Gs[g] > INT32_MAX ? INT32_MAX
                                                                        : Hkvs[h] * Gs[g]);
        d.block_size = bss[k];
        d.max_blocks_per_seq = mbss[m];
        d.num_blocks = 1024;
        d.variant = v;
        d.num_query_tokens = Ts[t];
        const int32_t S = sa_decode_num_splits(&d, windows[w]);
        const size_t ws = sa_decode_workspace_bytes(&d, windows[w]);
        if (S < 0) {
            CHECK(ws == 0, "invalid dims size a workspace (%zu)", ws);
            continue;
        }
        CHECK(S >= 1, "S = %d", S);
        /* the sizes must fit the fake device region for a launch check */
        if (ws > ((size_t)1 << 40)) continue;
        const int before = sa_test_launch_count();
        const int st = call_attention(&d, windows[w], -1, -1, ws);
        if (st == SA_ERR_HIP) {
            ++launched;
            CHECK(sa_test_launch_count() > before, "launch not reached");
        } else {
            /* a grid the launch cannot take is refused, never launched */
            CHECK(st < 0 && sa_test_launch_count() == before,
                  "B=%d Hkv=%d G=%d bs=%d mbs=%d W=%d v=%d T=%d: status %d", d.num_seqs,
                  d.num_kv_heads, Gs[g], d.block_size, d.max_blocks_per_seq, windows[w], v,
                  d.num_query_tokens, st);
        }
    }
    CHECK(launched > 1000, "only %d sweep configurations reached a launch", launched);
}

int main(void) {
    /* 1 TiB of address space with no access: the library may compute device
       addresses in it but never touch them */
    g_dev = mmap(NULL, (size_t)1 << 40, PROT_NONE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE,
                 -1, 0);
    if (g_dev == MAP_FAILED) {
        perror("mmap");
        return 2;
    }
    entry_points();
    planner_sweep();
    if (g_fail) {
        fprintf(stderr, "%d of %d checks failed\n", g_fail, g_checks);
        return 1;
    }
    printf("ok %d checks, %d launches reached\n", g_checks, sa_test_launch_count());
    return 0;
}
