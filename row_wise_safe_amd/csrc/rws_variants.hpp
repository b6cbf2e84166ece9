// rws_variants.hpp -- the compiled variants of each kernel family (X-macro
// lists shared by the plain and the masked launchers; the dispatcher indexes
// the resulting tables in rws_launch.hpp).
#pragma once

// (G lanes per row, K granules per lane, U row sets per wave); the last four
// serve the masked form and rows that are not line-aligned (two or three
// granules per lane on less than a wave)
#define RWS_WAVE_ROW_VARIANTS(X) \
    X(4, 1, 1)                   \
    X(8, 1, 1)                   \
    X(16, 1, 1)                  \
    X(32, 1, 1)                  \
    X(64, 1, 1)                  \
    X(64, 1, 2)                  \
    X(64, 2, 1)                  \
    X(64, 4, 1)                  \
    X(64, 8, 1)                  \
    X(8, 2, 1)                   \
    X(16, 2, 1)                  \
    X(32, 2, 1)                  \
    X(32, 3, 1)

// (threads, register granules per thread, LDS granules per thread): one
// granule per thread for launches with few waves, 2-5 for many rows (the
// dispatcher takes the shape with the fewest idle slots; these are the ones
// that rule can reach), and the shapes for long rows.
#define RWS_ONEPASS_VARIANTS(X)                                              \
    X(128, 1, 0) X(192, 1, 0) X(256, 1, 0) X(320, 1, 0) X(384, 1, 0)        \
    X(512, 1, 0) X(640, 1, 0) X(768, 1, 0) X(1024, 1, 0)                    \
    X(128, 2, 0) X(192, 2, 0) X(256, 2, 0) X(320, 2, 0) X(384, 2, 0)        \
    X(512, 2, 0) X(768, 2, 0) X(1024, 2, 0)                                 \
    X(64, 3, 0) X(192, 3, 0) X(384, 3, 0) X(1024, 3, 0)                     \
    X(1024, 4, 0) X(64, 5, 0)                                               \
    X(1024, 6, 0) X(1024, 8, 0) X(1024, 8, 8)

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
