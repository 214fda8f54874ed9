"""Shrunken variants of the five workloads (same formats, routers and options,
smaller E/H/F/T) so that brute force and parity run in seconds."""
import gen

SHRUNK = {
    "tiny": gen.CONFIGS["tiny"],
    "qwen3.6-35b-a3b": gen.CONFIGS["qwen3.6-35b-a3b"].with_(name="qwen-shrunk", E=16, H=512,
                                                            F=256, T=3),
    "gpt-oss-20b": gen.CONFIGS["gpt-oss-20b"].with_(name="gptoss-shrunk", E=8, H=320, F=288,
                                                    T=3),
    "deepseek-v4-flash": gen.CONFIGS["deepseek-v4-flash"].with_(name="dsv4-shrunk", E=16,
                                                                H=512, F=256, T=5),
    "kimi-k2": gen.CONFIGS["kimi-k2"].with_(name="kimi-shrunk", E=24, H=768, F=256, T=7),
}
