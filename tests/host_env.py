"""Environment for the compilers and programs that CPU tests start as child processes."""
import os


def child_env() -> dict:
    """A copy of this process's environment in which, under tests/sanitize_host.py (which sets
    BSQ_TEST_SANITIZED=1 and preloads the ASan runtime for the instrumented libraries), the
    ASan runtime is taken out of LD_PRELOAD: the children are not instrumented.  Every other
    LD_PRELOAD entry, and every entry outside a sanitizer run, is left as it is."""
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD")
    if pre and env.get("BSQ_TEST_SANITIZED") == "1":
        keep = [p for p in pre.replace(":", " ").split() if not os.path.basename(p).startswith("libclang_rt.asan")]
        if keep:
            env["LD_PRELOAD"] = " ".join(keep)
        else:
            del env["LD_PRELOAD"]
    return env
