// Token-file data loader (host only).
//
// The pages' data files are raw byte streams of int32 GPT-2 token ids with no
// header (ujoy.net article "徒手用 1000 行 C 语言实现", section "训练过程": the
// tiny_shakespeare_{train,val}.bin files, 305,260 and 32,768 tokens).  A batch
// is B consecutive sequences of T tokens read from one contiguous window of
// B*T + 1 ids: tokens = window[0 .. B*T), targets = window[1 .. B*T] (each
// sequence's targets are its tokens shifted by one; the last target of a
// sequence is the first token of the next).  Successive batches advance by
// B*T ids; when fewer than B*T + 1 ids remain the position returns to the
// start.  num_batches = floor(num_tokens / (B*T)), which gives the printed
// 1192 train and 128 val batches at B*T = 256.
//
// The file is read with one pread per batch (nothing is held in memory
// beyond one window), so files far larger than host memory work.
#include <errno.h>
#include <stdarg.h>
#include <fcntl.h>
#include <stdint.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdio>
#include <new>
#include <vector>

#include "gpt2.h"

int gpt2_set_error(int code, const char* msg);  // host.cpp

struct gpt2_loader {
    int fd = -1;
    int B = 0, T = 0;
    int64_t ntok = 0;  // ids in the file
    int64_t pos = 0;   // next window start, in ids
    std::vector<int32_t> win;
};

namespace {

int lfail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int lfail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return gpt2_set_error(code, buf);
}

}  // namespace

extern "C" {

int gpt2_loader_open(const char* path, int B, int T, gpt2_loader** out) {
    if (!path || !out) return lfail(GPT2_EINVAL, "NULL argument");
    *out = nullptr;
    if (B <= 0 || T <= 0 || (int64_t)B * T > (1 << 30))
        return lfail(GPT2_EINVAL, "B=%d T=%d out of range", B, T);
    const int fd = ::open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return lfail(GPT2_EINVAL, "cannot open %s: %s", path, strerror(errno));
    struct stat st;
    if (fstat(fd, &st) != 0) {
        ::close(fd);
        return lfail(GPT2_EINVAL, "cannot stat %s: %s", path, strerror(errno));
    }
    if (!S_ISREG(st.st_mode)) {
        ::close(fd);
        return lfail(GPT2_EINVAL, "%s is not a regular file", path);
    }
    if (st.st_size % 4 != 0) {
        ::close(fd);
        return lfail(GPT2_EINVAL, "%s: %lld bytes is not a whole number of int32 ids", path,
                     (long long)st.st_size);
    }
    const int64_t ntok = st.st_size / 4;
    if (ntok < (int64_t)B * T + 1) {
        ::close(fd);
        return lfail(GPT2_EINVAL, "%s holds %lld ids, fewer than one batch window (%lld)", path,
                     (long long)ntok, (long long)B * T + 1);
    }
    gpt2_loader* L = new (std::nothrow) gpt2_loader;
    if (!L) {
        ::close(fd);
        return lfail(GPT2_ENOMEM, "loader allocation failed");
    }
    L->fd = fd;
    L->B = B;
    L->T = T;
    L->ntok = ntok;
    try {
        L->win.resize((size_t)B * T + 1);
    } catch (...) {
        ::close(fd);
        delete L;
        return lfail(GPT2_ENOMEM, "loader window allocation failed");
    }
    *out = L;
    return GPT2_OK;
}

int64_t gpt2_loader_num_tokens(const gpt2_loader* L) { return L ? L->ntok : -1; }

int64_t gpt2_loader_num_batches(const gpt2_loader* L) {
    return L ? L->ntok / ((int64_t)L->B * L->T) : -1;
}

int gpt2_loader_next(gpt2_loader* L, int32_t* tokens, int32_t* targets) {
    if (!L || !tokens || !targets) return lfail(GPT2_EINVAL, "NULL argument");
    const int64_t bt = (int64_t)L->B * L->T;
    if (L->pos + bt + 1 > L->ntok) L->pos = 0;
    const size_t want = (size_t)(bt + 1) * 4;
    size_t got = 0;
    char* dst = reinterpret_cast<char*>(L->win.data());
    while (got < want) {
        const ssize_t r = pread(L->fd, dst + got, want - got, (off_t)(L->pos * 4 + (int64_t)got));
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return lfail(GPT2_EINVAL, "token file read failed at id %lld", (long long)L->pos);
        got += (size_t)r;
    }
    memcpy(tokens, L->win.data(), (size_t)bt * 4);
    memcpy(targets, L->win.data() + 1, (size_t)bt * 4);
    L->pos += bt;
    return GPT2_OK;
}

int gpt2_loader_reset(gpt2_loader* L) {
    if (!L) return lfail(GPT2_EINVAL, "NULL argument");
    L->pos = 0;
    return GPT2_OK;
}

void gpt2_loader_close(gpt2_loader* L) {
    if (!L) return;
    if (L->fd >= 0) ::close(L->fd);
    delete L;
}

}  // extern "C"
