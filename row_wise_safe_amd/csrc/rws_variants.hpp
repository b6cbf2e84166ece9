// rws_variants.hpp -- the compiled variants of each kernel family (X-macro
// lists shared by the plain and the masked launchers; the dispatcher indexes
// the resulting tables in rws_launch.hpp).
#pragma once

// (G lanes per row, K granules per lane, U row sets per wave)
#define RWS_WAVE_ROW_VARIANTS(X) \
    X(4, 1, 1)                   \
    X(8, 1, 1)                   \
    X(16, 1, 1)                  \
    X(32, 1, 1)                  \
    X(64, 1, 1)                  \
    X(64, 1, 2)                  \
    X(64, 2, 1)                  \
    X(64, 4, 1)                  \
    X(64, 8, 1)

// (threads, register granules per thread, LDS granules per thread)
#define RWS_ONEPASS_VARIANTS(X) \
    X(256, 2, 0)                \
    X(192, 3, 0)                \
    X(256, 3, 0)                \
    X(256, 4, 0)                \
    X(512, 4, 0)                \
    X(1024, 4, 0)               \
    X(1024, 8, 0)               \
    X(1024, 8, 8)

// (threads, granules per thread per batch)
#define RWS_TWO_PASS_VARIANTS(X) \
    X(256, 4)                    \
    X(512, 4)                    \
    X(1024, 2)                   \
    X(1024, 4)

// split-k (threads, granules per thread per chunk): the two-launch and the
// ordered single-launch forms share the list, so the dispatcher's chunking
// applies to both.
#define RWS_SPLITK_VARIANTS(X) \
    X(256, 2)                  \
    X(256, 4)                  \
    X(256, 8)                  \
    X(512, 8)
